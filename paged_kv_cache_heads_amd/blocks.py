"""Python binding of the host block manager (include/pa_blocks.h).

Argument marshalling only: every method calls the C entry point of the same
name on host numpy arrays and raises PAError on a non-zero status (status
PA_ERR_NO_BLOCKS = 7 when the pool is short: the call changed nothing).
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from . import PAError

PA_ERR_NO_BLOCKS = 7
PA_ERR_NOT_FOUND = 8


def _check(fn, status):
    if status != 0:
        raise PAError(fn, status)


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def xxh64(data: bytes, seed: int = 0) -> int:
    buf = ctypes.create_string_buffer(bytes(data), len(data) + 1)
    return int(_lib.load().pa_xxh64(buf, len(data), seed))


class BlockManager:
    """Pool of num_blocks cache blocks of block_size tokens (order: initial free-list order)."""

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self._lib = _lib.load()
        self.block_size = block_size
        self.num_blocks = num_blocks
        h = ctypes.c_void_p()
        arr = None if order is None else _i32(order)
        _check("pa_bm_create", self._lib.pa_bm_create(num_blocks, block_size,
                                                      None if arr is None else arr.ctypes.data, ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_bm_destroy(h)
            self._h = None

    def allocate(self, seq_id: int, tokens) -> int:
        t = _i32(tokens)
        cached = ctypes.c_int32(0)
        _check("pa_bm_allocate", self._lib.pa_bm_allocate(self._h, int(seq_id), t.ctypes.data if t.size else None,
                                                          int(t.size), ctypes.byref(cached)))
        return cached.value

    def append(self, seq_id: int, token: int) -> None:
        _check("pa_bm_append", self._lib.pa_bm_append(self._h, int(seq_id), int(token)))

    def append_batch(self, seq_ids, tokens) -> int:
        """Append tokens[i] to seq_ids[i] in order; returns how many were appended
        (raises PAError at the first failure, after the earlier appends)."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        t = _i32(tokens)
        done = ctypes.c_int32(0)
        st = self._lib.pa_bm_append_batch(self._h, ids.ctypes.data, t.ctypes.data, int(ids.size), ctypes.byref(done))
        _check("pa_bm_append_batch", st)
        return done.value

    def free_seq(self, seq_id: int) -> None:
        _check("pa_bm_free", self._lib.pa_bm_free(self._h, int(seq_id)))

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def length(self, seq_id: int) -> int:
        return int(self._lib.pa_bm_seq_len(self._h, int(seq_id)))

    def table(self, seq_id: int):
        n = ctypes.c_int32(0)
        cap = max(1, -(-max(self.length(seq_id), 0) // self.block_size))
        out = np.empty(cap, dtype=np.int32)
        _check("pa_bm_block_table", self._lib.pa_bm_block_table(self._h, int(seq_id), out.ctypes.data, cap,
                                                                ctypes.byref(n)))
        return out[:n.value].tolist()

    def free_list(self):
        n = ctypes.c_int32(0)
        out = np.empty(max(1, self.num_blocks), dtype=np.int32)
        _check("pa_bm_free_list", self._lib.pa_bm_free_list(self._h, out.ctypes.data, self.num_blocks,
                                                            ctypes.byref(n)))
        return out[:n.value].tolist()

    def ref(self, block: int) -> int:
        return int(self._lib.pa_bm_block_ref(self._h, int(block)))

    def decode_metadata(self, seq_ids, width: int):
        """(block_tables [S, width], context_lens [S], slot_mapping [S]) as int32 arrays."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        s = int(ids.size)
        bt = np.empty((s, width), dtype=np.int32)
        cl = np.empty(s, dtype=np.int32)
        sm = np.empty(s, dtype=np.int32)
        _check("pa_bm_decode_metadata", self._lib.pa_bm_decode_metadata(
            self._h, ids.ctypes.data, s, int(width), bt.ctypes.data, cl.ctypes.data, sm.ctypes.data))
        return bt, cl, sm

    def prefill_metadata(self, seq_ids, num_cached, width: int):
        """(block_tables [S, width], cu_seqlens_q [S+1], cu_seqlens_k [S+1], slot_mapping [Tq])."""
        ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        nc = _i32(num_cached)
        s = int(ids.size)
        total = sum(self.length(i) - int(c) for i, c in zip(ids.tolist(), nc.tolist()))
        bt = np.empty((s, width), dtype=np.int32)
        cq = np.empty(s + 1, dtype=np.int32)
        ck = np.empty(s + 1, dtype=np.int32)
        sm = np.empty(max(total, 1), dtype=np.int32)
        _check("pa_bm_prefill_metadata", self._lib.pa_bm_prefill_metadata(
            self._h, ids.ctypes.data, nc.ctypes.data, s, int(width), bt.ctypes.data, cq.ctypes.data, ck.ctypes.data,
            sm.ctypes.data, total))
        return bt, cq, ck, sm[:total]
