"""Comparison helpers for GPU-vs-oracle parity (test code only)."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import tensors

# Attention outputs pass element-wise iff |got - ref| <= max(ATOL, RTOL * |ref|):
# the absolute bound governs where |ref| < 0.5, the relative bound above it.
ATOL = 1e-2
RTOL = 2e-2


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def attention_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    big = np.abs(ref) >= 0.5
    return {
        "max_abs": float(np.nanmax(err)) if err.size else 0.0,
        "max_rel_ref_ge_0.5": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "n": int(err.size),
    }


def assert_attention_close(got_t: torch.Tensor, ref: np.ndarray, what: str = "") -> dict:
    got = bf16_to_f64(got_t)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output at {np.argwhere(~np.isfinite(got))[:5]}"
    err = np.abs(got - ref)
    bound = np.maximum(ATOL, RTOL * np.abs(ref))
    bad = err > bound
    stats = attention_errors(got, ref)
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance; first {idx}: "
                             f"got {got[idx]} ref {ref[idx]}; {stats}")
    return stats


class Compact:
    """Host copy of the blocks some sequences use, with their tables renumbered.

    The oracle's results do not depend on which physical blocks hold a
    sequence (pinned by the oracle's permutation-invariance check), so the
    oracle can run on this small copy of a large pool.
    """

    def __init__(self, batch, seqs, extra_blocks=()):
        wl = batch.wl
        bs = wl.block_size
        used = []
        for s in seqs:
            n = int(wl.kv_lens()[s])
            used.extend(int(x) for x in wl.block_tables[s, :-(-n // bs)])
        used.extend(int(x) for x in extra_blocks)
        self.blocks = sorted(set(used))
        self.index = {b: i for i, b in enumerate(self.blocks)}
        idx = torch.tensor(self.blocks, dtype=torch.int64, device=batch.k_cache.device)
        self.k = tensors.to_u16(batch.k_cache[idx])
        self.v = tensors.to_u16(batch.v_cache[idx])
        self.seqs = list(seqs)
        self.tables = np.full((len(seqs), wl.block_tables.shape[1]), -1, dtype=np.int64)
        for i, s in enumerate(seqs):
            for j, b in enumerate(wl.block_tables[s]):
                if b >= 0 and int(b) in self.index:
                    self.tables[i, j] = self.index[int(b)]

    def remap_slot(self, slot: int, bs: int) -> int:
        if slot < 0 or slot // bs not in self.index:
            return -1  # padding, or a token of a sequence outside this copy
        return self.index[slot // bs] * bs + slot % bs

    def store(self, k_new: np.ndarray, v_new: np.ndarray, slots, bs: int):
        """The oracle's store applied to this copy (slots of the full pool)."""
        remapped = np.array([self.remap_slot(int(s), bs) for s in slots], dtype=np.int64)
        self.k, self.v = oracle.store_kvcache(k_new, v_new, remapped, self.k, self.v)
