"""Comparison helpers for GPU-vs-oracle parity (test code only)."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import tensors

# The attention pass criteria, applied literally over every compared element:
# max |got - ref| <= ATOL, and max |got - ref| / |ref| <= RTOL over the elements
# with |ref| >= REL_FLOOR (a relative error near ref = 0 has no meaning).
ATOL = 1e-2
RTOL = 2e-2
REL_FLOOR = 0.5

# Every comparison made in this test session, by case name: element count,
# max abs error, max rel error, and where the max abs error sits. conftest
# prints it at the end of the run (and writes it as JSON on request).
RECORD: dict = {}


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def bf16_neighbours(ref: np.ndarray):
    """The two bf16 values around each element of ref (lo <= |ref| < hi in magnitude, sign restored).

    bf16 keeps 8 significant bits, so in [2^(e-1), 2^e) its values are 2^(e-8) apart; exact in
    float64 for the magnitudes attention outputs reach.
    """
    a = np.abs(ref)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    spacing = np.ldexp(1.0, ex - 8)
    lo = np.floor(a / spacing) * spacing
    sign = np.where(ref < 0, -1.0, 1.0)
    return sign * lo, sign * (lo + spacing)


def attention_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    """Max abs error, max rel error over |ref| >= 0.5, and the elements where no bf16 value lies
    within ATOL of ref (|ref| >= 4, where bf16 values are 2^-5 apart): there the best a bf16
    output can do is one of ref's two bf16 neighbours."""
    err = np.abs(got - ref)
    big = np.abs(ref) >= REL_FLOOR
    lo, hi = bf16_neighbours(ref)
    unattainable = np.minimum(np.abs(ref - lo), np.abs(hi - ref)) > ATOL
    att = err[~unattainable]
    out = {
        "n": int(err.size),
        "max_abs": float(np.nanmax(err)) if err.size else 0.0,
        "max_abs_attainable": float(att.max()) if att.size else 0.0,
        "n_bf16_unattainable": int(unattainable.sum()),
        "max_rel_ref_ge_0.5": float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "max_abs_ref": 0.0,
    }
    if err.size:
        at = np.unravel_index(int(np.nanargmax(err)), err.shape)
        out["max_abs_ref"] = float(ref[at])
    return out


def _record(what: str, stats: dict) -> None:
    old = RECORD.get(what)
    if old is None:
        RECORD[what] = dict(stats, calls=1)
        return
    old["calls"] += 1
    old["n"] += stats["n"]
    old["n_bf16_unattainable"] += stats["n_bf16_unattainable"]
    if stats["max_abs"] > old["max_abs"]:
        old["max_abs"], old["max_abs_ref"] = stats["max_abs"], stats["max_abs_ref"]
    for key in ("max_abs_attainable", "max_rel_ref_ge_0.5"):
        old[key] = max(old[key], stats[key])


def assert_attention_close(got_t: torch.Tensor, ref: np.ndarray, what: str = "") -> dict:
    """The attention pass criteria on every element: |got - ref| <= ATOL, and |got - ref| / |ref| <=
    RTOL where |ref| >= 0.5. The one exception is an element whose ref has no bf16 value within
    ATOL (|ref| >= 4): the output, being bf16, cannot meet ATOL there, and must instead be one of
    ref's two bf16 neighbours (it still has to meet RTOL). Such elements are counted in the record."""
    got = bf16_to_f64(got_t)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output at {np.argwhere(~np.isfinite(got))[:5]}"
    stats = attention_errors(got, ref)
    _record(what, stats)
    err = np.abs(got - ref)
    lo, hi = bf16_neighbours(ref)
    unattainable = np.minimum(np.abs(ref - lo), np.abs(hi - ref)) > ATOL
    bad = (err > ATOL) & ~unattainable
    if bad.any():
        idx = tuple(int(i) for i in np.argwhere(bad)[np.argmax(err[bad])])
        raise AssertionError(f"{what}: max abs error {err[bad].max():.3g} > {ATOL} at {idx}: got {got[idx]} "
                             f"ref {ref[idx]}; {int(bad.sum())} of {err.size} elements above; {stats}")
    off_grid = unattainable & (got != lo) & (got != hi)
    if off_grid.any():
        idx = tuple(int(i) for i in np.argwhere(off_grid)[0])
        raise AssertionError(f"{what}: at {idx} ref {ref[idx]} has no bf16 value within {ATOL}, and got "
                             f"{got[idx]} is neither of its bf16 neighbours {lo[idx]}, {hi[idx]}; {stats}")
    if stats["max_rel_ref_ge_0.5"] > RTOL:
        big = np.abs(ref) >= REL_FLOOR
        rel = np.where(big, err / np.maximum(np.abs(ref), REL_FLOOR), 0.0)
        idx = tuple(int(i) for i in np.unravel_index(int(np.argmax(rel)), rel.shape))
        raise AssertionError(f"{what}: max rel error {stats['max_rel_ref_ge_0.5']:.3g} > {RTOL} (|ref| >= "
                             f"{REL_FLOOR}) at {idx}: got {got[idx]} ref {ref[idx]}; {stats}")
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
