"""pa_qk_norm_rope_store on the GPU against the fp64 oracle.

q and the stored K: element by element within the bf16 output bound (one
rounding to bf16, at most 2^-7 relative, plus 1e-4 absolute for fp32
cancellation in the rotation). V and every cache row that no valid slot names:
bit-exact.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401
from workloads import configs, rope, tensors
from workloads.bf16 import decode_f32

pytestmark = pytest.mark.gpu

RTOL, ATOL = 2.0 ** -7, 1e-4


def _close(got_bits, ref, what):
    got = decode_f32(got_bits).astype(np.float64)
    err = np.abs(got - ref)
    bound = RTOL * np.abs(ref) + ATOL
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside the bound, max err {err.max():.3e}"
    return float(err.max())


def _run(batch, positions, dev, *, eps=1e-6, max_position=40960, seed=0, slots=None, inplace=False):
    wl = batch.wl
    hq, hkv, d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    rng = np.random.default_rng(seed)
    qw, kw = rope.norm_weight(rng, d), rope.norm_weight(rng, d)
    table = rope.cos_sin_table(max_position, d, base=1.0e6)
    to_dev = lambda a, dt: torch.as_tensor(np.ascontiguousarray(a)).to(dev).view(dt)  # noqa: E731
    qw_t, kw_t = to_dev(qw.view(np.int16), torch.bfloat16), to_dev(kw.view(np.int16), torch.bfloat16)
    table_t = torch.as_tensor(table).to(dev)
    pos_t = torch.as_tensor(np.asarray(positions, np.int32)).to(dev)
    slot_t = batch.slot_mapping if slots is None else torch.as_tensor(np.asarray(slots, np.int32)).to(dev)
    qkv_bits = tensors.to_u16(batch.qkv)
    slots_h = slot_t.cpu().numpy()
    cap = wl.num_blocks * wl.block_size
    valid = (slots_h >= 0) & (slots_h < cap)
    touched = sorted({int(s) // wl.block_size for s in slots_h[valid]})
    idx = torch.tensor(touched, dtype=torch.int64, device=dev)
    k_before, v_before = tensors.to_u16(batch.k_cache[idx]), tensors.to_u16(batch.v_cache[idx])
    mask = torch.ones(wl.num_blocks, dtype=torch.bool, device=dev)
    mask[idx] = False
    snap_k, snap_v = batch.k_cache[mask].clone(), batch.v_cache[mask].clone()

    q_out = batch.q if inplace else None
    q_out = pa.pa_qk_norm_rope_store(batch.qkv, qw_t, kw_t, eps, table_t, pos_t, batch.k_cache, batch.v_cache,
                                     slot_t, hq, q_out=q_out)
    torch.cuda.synchronize()

    clamped = np.clip(np.asarray(positions, np.int64), 0, max_position - 1)
    ref_q, ref_k, ref_v = oracle.qk_norm_rope(qkv_bits, clamped, table, qw, kw, eps, hq, hkv)
    err_q = _close(tensors.to_u16(q_out), ref_q, f"{wl.name} q")

    # stored rows: K within the bound, V bit-exact; the rest of each touched block unchanged
    k_after, v_after = tensors.to_u16(batch.k_cache[idx]), tensors.to_u16(batch.v_cache[idx])
    pos_of = {b: i for i, b in enumerate(touched)}
    written = np.zeros(k_after.shape[:2], dtype=bool)
    err_k = 0.0
    for t in np.nonzero(valid)[0]:
        s = int(slots_h[t])
        bi, r = pos_of[s // wl.block_size], s % wl.block_size
        written[bi, r] = True
        err_k = max(err_k, _close(k_after[bi, r], ref_k[t], f"{wl.name} k token {t}"))
        assert np.array_equal(v_after[bi, r], ref_v[t]), f"{wl.name} v token {t}"
    assert np.array_equal(k_after[~written], k_before[~written])
    assert np.array_equal(v_after[~written], v_before[~written])
    assert torch.equal(batch.k_cache[mask].view(torch.int16), snap_k.view(torch.int16))
    assert torch.equal(batch.v_cache[mask].view(torch.int16), snap_v.view(torch.int16))
    return err_q, err_k


@pytest.mark.parametrize("hq,hkv", [(16, 8), (8, 8), (32, 8), (32, 4), (64, 8)])
def test_norm_rope_heads(dev, hq, hkv):
    announce(f"norm_rope heads {hq}/{hkv}")
    wl = configs.prefill_workload("nr-heads", [1, 5, 37, 130], 0, hq, hkv, 16, seed=31)
    _run(tensors.materialize(wl, dev), wl.store_pos, dev, seed=1)


def test_norm_rope_prefill_batch(dev):
    # the varlen prefill batch: 15815 tokens, Hq 16, Hkv 8, positions 0 .. len - 1
    announce("norm_rope varlen prefill batch")
    wl = configs.config3()
    _run(tensors.materialize(wl, dev), wl.store_pos, dev, seed=2)


def test_norm_rope_prefix_batch_positions_past_prefix(dev):
    announce("norm_rope prefix batch (positions 1024 ..)")
    wl = configs.config4()
    _run(tensors.materialize(wl, dev), wl.store_pos, dev, seed=3)


def test_norm_rope_decode_batch(dev):
    # decode: one token per sequence at position L - 1; sequences of length 0 have slot -1
    announce("norm_rope decode batch")
    wl = configs.config2()
    batch = tensors.materialize(wl, dev)
    pos = np.zeros(wl.num_seqs, np.int64)
    pos[wl.store_seq] = wl.store_pos
    _run(batch, pos, dev, seed=4)


def test_norm_rope_skipped_slots_and_clamped_positions(dev):
    announce("norm_rope skipped slots, clamped positions, eps 0.1")
    wl = configs.prefill_workload("nr-edge", [7, 50], 0, 16, 8, 8, seed=32)
    batch = tensors.materialize(wl, dev)
    slots = wl.slot_mapping.copy()
    cap = wl.num_blocks * wl.block_size
    slots[0], slots[3], slots[10] = -1, cap, cap + 1000  # negative and past the pool: nothing stored
    pos = wl.store_pos.astype(np.int64).copy()
    pos[1], pos[2] = -5, 10 ** 6  # clamped into [0, max_position)
    _run(batch, pos, dev, eps=0.1, max_position=64, seed=5, slots=slots)


def test_norm_rope_in_place_and_strided_rows(dev):
    # q_out is the q columns of qkv itself; qkv rows padded past the heads
    announce("norm_rope in place, padded qkv rows")
    wl = configs.prefill_workload("nr-inplace", [3, 64, 65], 0, 16, 8, 8, seed=33)
    batch = tensors.materialize(wl, dev)
    t, w = batch.qkv.shape
    wide = torch.zeros((t, w + 64), dtype=torch.bfloat16, device=dev)
    wide[:, :w] = batch.qkv
    batch.qkv = wide[:, :w]
    batch.q = batch.qkv[:, :16 * 128].unflatten(1, (16, 128))
    _run(batch, wl.store_pos, dev, seed=6, inplace=True)


def test_norm_rope_empty(dev):
    announce("norm_rope zero tokens")
    wl = configs.prefill_workload("nr-empty", [3], 0, 16, 8, 4, seed=34)
    batch = tensors.materialize(wl, dev)
    empty = batch.qkv[:0]
    pos = torch.zeros(0, dtype=torch.int32, device=dev)
    table = torch.zeros((8, 128), dtype=torch.float32, device=dev)
    w = torch.ones(128, dtype=torch.bfloat16, device=dev)
    out = pa.pa_qk_norm_rope_store(empty, w, w, 1e-6, table, pos, batch.k_cache, batch.v_cache,
                                   batch.slot_mapping[:0], 16)
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 128)
