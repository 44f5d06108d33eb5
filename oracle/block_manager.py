"""Plain Python model of the host-side KV block manager (prefix caching).

TEST INFRASTRUCTURE ONLY (see the package docstring). The C++ block manager
in the library is checked against this model operation by operation; they
share no code.

What it does (page "nano-vLLM 最小化vLLM重新实现", section 3 "块管理器": a pool
of fixed-size KV blocks handed out from a free list, each block carrying a
reference count and a hash; allocation reuses cached prefix blocks whose hash
matches and allocates only the rest; blocks are hashed per token block with
xxhash; preemption frees a sequence's blocks; page at hotelren.com/news/2273631,
section 2.2: each sequence's block list is its page table and freed blocks
return to the pool; section 4.4: a cached prefix's KV is reused and only the
remainder computed).

Readings where the pages are silent (listed in the design doc):

* A full block's hash chains through the prefix: h_i = xxh64(token ids of
  block i as little-endian int32, seed = h_{i-1}), h_{-1} = 0, so equal
  blocks after different prefixes do not match. Only full blocks are hashed.
* A hash hit also compares the block's token ids (a collision is a miss).
  Matching stops at the first miss. At most (n - 1) // block_size blocks of an
  n-token prompt come from the cache, so at least one token is computed.
* The free list is a queue: blocks are taken from the front; a finished (or
  preempted) sequence returns its blocks to the back, last block first. A
  freed block keeps its hash, so a later prompt can still hit it, until it is
  taken for new content. A block's hash is registered in the cache only if
  that hash is not already there.
* An allocation or append that lacks blocks fails and changes nothing (the
  scheduler then preempts).
"""

from __future__ import annotations

import numpy as np
import xxhash


class NoBlocks(Exception):
    pass


def block_hash(tokens, seed: int) -> int:
    """xxh64 of the block's token ids (int32, little-endian), chained through seed."""
    return xxhash.xxh64_intdigest(np.asarray(tokens, dtype="<i4").tobytes(), seed=seed)


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.block_size = block_size
        self.free = list(range(num_blocks)) if order is None else [int(b) for b in order]
        self.ref = [0] * num_blocks
        self.hash = [None] * num_blocks      # hash of the content a block holds, or None
        self.content = [None] * num_blocks   # (parent hash, token tuple) of a hashed block
        self.cache = {}                      # hash -> block
        self.seqs = {}                       # seq id -> dict(table, len, last_hash, partial)

    # -- helpers --
    def _take(self):
        b = self.free.pop(0)
        h = self.hash[b]
        if h is not None and self.cache.get(h) == b:
            del self.cache[h]
        self.hash[b] = None
        self.content[b] = None
        self.ref[b] = 1
        return b

    def _register(self, b, h, parent, toks):
        self.hash[b] = h
        self.content[b] = (parent, tuple(toks))
        if h not in self.cache:
            self.cache[h] = b

    # -- operations --
    def allocate(self, seq_id, tokens) -> int:
        """Blocks for a new sequence's prompt; returns how many prompt tokens were cached."""
        assert seq_id not in self.seqs
        bs = self.block_size
        toks = [int(t) for t in tokens]
        n = len(toks)
        nblocks = -(-n // bs)
        hits, h = [], 0
        for i in range((n - 1) // bs if n > 0 else 0):
            blk = toks[i * bs:(i + 1) * bs]
            hi = block_hash(blk, h)
            b = self.cache.get(hi)
            if b is None or self.content[b] != (h, tuple(blk)):
                break
            hits.append(b)
            h = hi
        from_free = sum(1 for b in hits if self.ref[b] == 0)
        if nblocks - len(hits) + from_free > len(self.free):
            raise NoBlocks()
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
        table = list(hits)
        for i in range(len(hits), nblocks):
            b = self._take()
            table.append(b)
            if (i + 1) * bs <= n:
                blk = toks[i * bs:(i + 1) * bs]
                hi = block_hash(blk, h)
                self._register(b, hi, h, blk)
                h = hi
        full = n // bs
        self.seqs[seq_id] = {"table": table, "len": n, "last_hash": h if full else 0,
                             "partial": toks[full * bs:]}
        return len(hits) * bs

    def append(self, seq_id, token) -> None:
        """One more token (decode); takes a new block when the last one is full."""
        s = self.seqs[seq_id]
        bs = self.block_size
        if s["len"] % bs == 0:
            if not self.free:
                raise NoBlocks()
            s["table"].append(self._take())
        s["partial"].append(int(token))
        s["len"] += 1
        if s["len"] % bs == 0:
            b = s["table"][-1]
            hi = block_hash(s["partial"], s["last_hash"])
            self._register(b, hi, s["last_hash"], s["partial"])
            s["last_hash"] = hi
            s["partial"] = []

    def free_seq(self, seq_id) -> None:
        """Release a finished or preempted sequence's blocks (last block first)."""
        s = self.seqs.pop(seq_id)
        for b in reversed(s["table"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- queries --
    def table(self, seq_id):
        return list(self.seqs[seq_id]["table"])

    def length(self, seq_id) -> int:
        return self.seqs[seq_id]["len"]

    def num_free(self) -> int:
        return len(self.free)

    def slot(self, seq_id, pos: int) -> int:
        t = self.seqs[seq_id]["table"]
        return t[pos // self.block_size] * self.block_size + pos % self.block_size
