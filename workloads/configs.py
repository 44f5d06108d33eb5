"""Seeded synthetic workloads: lengths, block tables, slot mappings, cu_seqlens.

Host-side metadata only (numpy). What a block manager and scheduler would hand
to the kernels, built from seeds: a shuffled pool of physical blocks, each
sequence taking consecutive entries of the shuffle (page "nano-vLLM
最小化vLLM重新实现", section 3 "块管理器": fixed 256-token blocks from a free
pool; page at hotelren.com/news/2273631, section 2.2: a per-sequence list of
physical blocks). No attention or store arithmetic lives here; the one piece of
paging bookkeeping (slot = block * block_size + row) is checked against the
oracle's own definition by tests/test_workloads.py.

The five standard workloads (shapes of the Qwen3-0.6B-sized models the pages
benchmark; lengths drawn like the pages' random request lengths):

  1 tiny decode      Hq 16, Hkv 8, 16 blocks, context lens {1, 37, 256, 300}
  2 decode           Hq 16, Hkv 8, 256 seqs, L ~ U{100..2048}, 4096-block pool
  3 varlen prefill   Hq 16, Hkv 8, 64 lengths ~ U{100..1024}, admitted in order
                     while the total stays <= 16384 tokens
  4 prefix prefill   Hq 16, Hkv 8, 32 seqs sharing a 1024-token prefix in 4
                     blocks, each adding m ~ U{128..512} tokens
  5 long decode      Hq 32, Hkv 8, 512 seqs, L log-uniform in [256, 32768],
                     164,794-block pool (60% of 288 GB at 1 MiB per K+V block)
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEAD_DIM = 128
BLOCK_SIZE = 256


@dataclass
class Workload:
    name: str
    kind: str  # "decode" or "prefill"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    seed: int
    block_tables: np.ndarray            # [S, W] int32, -1 past each sequence's blocks
    slot_mapping: np.ndarray            # [T] int32, one per stored token
    store_seq: np.ndarray               # [T] sequence of each stored token
    store_pos: np.ndarray               # [T] position of each stored token in its sequence
    pre_len: np.ndarray                 # [S] positions holding data before the store
    context_lens: np.ndarray | None = None   # decode: [S], counts the stored token
    cu_seqlens_q: np.ndarray | None = None   # prefill: [S + 1]
    cu_seqlens_k: np.ndarray | None = None
    shared_prefix_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def num_tokens(self) -> int:
        return int(self.slot_mapping.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens is not None and len(self.context_lens) else 0

    @property
    def max_seqlen_q(self) -> int:
        return int(np.diff(self.cu_seqlens_q).max()) if self.cu_seqlens_q is not None and self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(np.diff(self.cu_seqlens_k).max()) if self.cu_seqlens_k is not None and self.num_seqs else 0

    def kv_lens(self) -> np.ndarray:
        """Keys each sequence attends over (decode: L; prefill: nk)."""
        if self.kind == "decode":
            return self.context_lens.astype(np.int64)
        return np.diff(self.cu_seqlens_k).astype(np.int64)


def blocks_for(n: int, block_size: int) -> int:
    return -(-int(n) // block_size)


def _slot(table_row, pos: int, block_size: int) -> int:
    return int(table_row[pos // block_size]) * block_size + pos % block_size


def _tables_from_perm(perm, needs, width, first=0, prefix=None):
    tables = np.full((len(needs), max(width, 1)), -1, dtype=np.int32)
    nxt = first
    for i, n in enumerate(needs):
        own = perm[nxt:nxt + n]
        nxt += n
        row = own if prefix is None else np.concatenate([prefix, own])
        tables[i, :len(row)] = row
    if nxt > len(perm):
        raise ValueError("block pool too small for the workload")
    return tables


def decode_workload(name, lengths, num_q_heads, num_kv_heads, num_blocks, seed, block_size=BLOCK_SIZE,
                    head_dim=HEAD_DIM) -> Workload:
    """Each sequence stores one new token at position L-1 and then attends to 0..L-1."""
    lengths = np.asarray(lengths, dtype=np.int32)
    perm = np.random.default_rng([seed, 1]).permutation(num_blocks).astype(np.int32)
    needs = [blocks_for(n, block_size) for n in lengths]
    tables = _tables_from_perm(perm, needs, max(needs) if needs else 1)
    has = lengths > 0
    seqs = np.nonzero(has)[0].astype(np.int32)
    pos = (lengths[has] - 1).astype(np.int32)
    slots = np.array([_slot(tables[b], p, block_size) for b, p in zip(seqs, pos)], dtype=np.int32)
    return Workload(name, "decode", num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, seed, tables, slots,
                    seqs, pos, np.maximum(lengths - 1, 0).astype(np.int32), context_lens=lengths)


def prefill_workload(name, new_lens, prefix_len, num_q_heads, num_kv_heads, num_blocks, seed,
                     block_size=BLOCK_SIZE, head_dim=HEAD_DIM) -> Workload:
    """Each sequence stores its new tokens at positions prefix_len .. prefix_len + m - 1.

    With prefix_len > 0 every sequence's table starts with the same
    prefix_len / block_size shared blocks (the cached prefix).
    """
    new_lens = np.asarray(new_lens, dtype=np.int32)
    if prefix_len % block_size:
        raise ValueError("the shared prefix must fill whole blocks")
    perm = np.random.default_rng([seed, 1]).permutation(num_blocks).astype(np.int32)
    n_prefix = prefix_len // block_size
    prefix = perm[:n_prefix]
    needs = [blocks_for(prefix_len + m, block_size) - n_prefix for m in new_lens]
    tables = _tables_from_perm(perm, needs, max(n + n_prefix for n in needs) if needs else 1, first=n_prefix,
                               prefix=prefix if n_prefix else None)
    seqs = np.repeat(np.arange(len(new_lens), dtype=np.int32), new_lens)
    pos = np.concatenate([np.arange(prefix_len, prefix_len + m, dtype=np.int32) for m in new_lens]) \
        if len(new_lens) else np.zeros(0, np.int32)
    slots = np.array([_slot(tables[b], p, block_size) for b, p in zip(seqs, pos)], dtype=np.int32)
    cu_q = np.concatenate([[0], np.cumsum(new_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(new_lens + prefix_len)]).astype(np.int32)
    return Workload(name, "prefill", num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, seed, tables,
                    slots, seqs, pos, np.full(len(new_lens), prefix_len, np.int32), cu_seqlens_q=cu_q,
                    cu_seqlens_k=cu_k, shared_prefix_blocks=prefix.astype(np.int32))


# ----------------------------------------------------------------------------- the five workloads


def config1(seed: int = 1) -> Workload:
    return decode_workload("cfg1-tiny-decode", [1, 37, 256, 300], 16, 8, 16, seed)


def config2(seed: int = 2) -> Workload:
    lens = np.random.default_rng([seed, 0]).integers(100, 2048, size=256, endpoint=True)
    return decode_workload("cfg2-qwen3-0.6b-decode", lens, 16, 8, 4096, seed)


def admitted_lengths(draws, budget: int):
    """Admit lengths in order while the running total stays within budget."""
    out, total = [], 0
    for n in draws:
        if total + int(n) > budget:
            break
        out.append(int(n))
        total += int(n)
    return out


def config3(seed: int = 3) -> Workload:
    draws = np.random.default_rng([seed, 0]).integers(100, 1024, size=64, endpoint=True)
    return prefill_workload("cfg3-varlen-prefill", admitted_lengths(draws, 16384), 0, 16, 8, 4096, seed)


def config4(seed: int = 4) -> Workload:
    m = np.random.default_rng([seed, 0]).integers(128, 512, size=32, endpoint=True)
    return prefill_workload("cfg4-prefix-prefill", m, 1024, 16, 8, 4096, seed)


CONFIG5_POOL_BLOCKS = int(0.6 * 288e9) // (2 * BLOCK_SIZE * 8 * HEAD_DIM * 2)  # 164,794


def log_uniform_lengths(rng, n, lo, hi):
    x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))).astype(np.int64)
    return np.clip(x, lo, hi)


def config5(seed: int = 5, num_blocks: int = CONFIG5_POOL_BLOCKS) -> Workload:
    lens = log_uniform_lengths(np.random.default_rng([seed, 0]), 512, 256, 32768)
    return decode_workload("cfg5-long-decode", lens, 32, 8, num_blocks, seed)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def get(k: int, seed: int | None = None) -> Workload:
    return CONFIGS[k]() if seed is None else CONFIGS[k](seed)
