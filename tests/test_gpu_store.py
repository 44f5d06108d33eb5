"""pa_store_kvcache on the GPU against the oracle's store: bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401
from tests.parity import Compact
from workloads import configs, tensors

pytestmark = pytest.mark.gpu


def _store_and_check(batch, dev):
    wl = batch.wl
    slots = batch.slot_mapping.cpu().numpy()
    bs = wl.block_size
    touched = sorted({int(s) // bs for s in slots if s >= 0})
    before = Compact(batch, [], extra_blocks=touched)
    snap_k, snap_v = batch.k_cache.clone(), batch.v_cache.clone()
    k_new, v_new = tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new)
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    torch.cuda.synchronize()
    # touched blocks: GPU bytes == oracle bytes (NaN filler included)
    before.store(k_new, v_new, slots, bs)
    idx = torch.tensor(touched, dtype=torch.int64, device=dev)
    assert np.array_equal(tensors.to_u16(batch.k_cache[idx]), before.k)
    assert np.array_equal(tensors.to_u16(batch.v_cache[idx]), before.v)
    # every other block unchanged
    mask = torch.ones(wl.num_blocks, dtype=torch.bool, device=dev)
    mask[idx] = False
    assert torch.equal(batch.k_cache[mask].view(torch.int16), snap_k[mask].view(torch.int16))
    assert torch.equal(batch.v_cache[mask].view(torch.int16), snap_v[mask].view(torch.int16))


@pytest.mark.parametrize("k,seed", [(1, None), (2, None), (3, None), (4, None), (1, 101), (3, 102), (4, 103)])
def test_store_config(dev, k, seed):
    announce(f"store config {k} seed {seed}")
    wl = configs.get(k, seed)
    _store_and_check(tensors.materialize(wl, dev), dev)


def test_store_config5_pool(dev):
    announce("store config 5 (161 GiB pool)")
    wl = configs.config5()
    batch = tensors.materialize(wl, dev)
    slots = batch.slot_mapping.cpu().numpy()
    bs = wl.block_size
    touched = sorted({int(s) // bs for s in slots if s >= 0})
    before = Compact(batch, [], extra_blocks=touched)
    k_new, v_new = tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new)
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    torch.cuda.synchronize()
    before.store(k_new, v_new, slots, bs)
    idx = torch.tensor(touched, dtype=torch.int64, device=dev)
    assert np.array_equal(tensors.to_u16(batch.k_cache[idx]), before.k)
    assert np.array_equal(tensors.to_u16(batch.v_cache[idx]), before.v)


def test_store_padding_and_small_blocks(dev):
    announce("store padding slots, block_size 64, odd token count")
    wl = configs.prefill_workload("pad", [3, 70, 1], 0, 4, 2, 12, seed=7, block_size=64)
    batch = tensors.materialize(wl, dev)
    slots = batch.slot_mapping.clone()
    slots[[0, 5, 40]] = -1  # padded tokens are skipped
    batch.slot_mapping = slots
    kc0 = tensors.to_u16(batch.k_cache)
    vc0 = tensors.to_u16(batch.v_cache)
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, slots)
    torch.cuda.synchronize()
    kref, vref = oracle.store_kvcache(tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new),
                                      slots.cpu().numpy(), kc0, vc0)
    assert np.array_equal(tensors.to_u16(batch.k_cache), kref)
    assert np.array_equal(tensors.to_u16(batch.v_cache), vref)


@pytest.mark.parametrize("hkv", [2, 3])
def test_store_slots_past_the_cache(dev, hkv):
    # slots at or past num_blocks * block_size store nothing (both kernel layouts: 2 kv heads take whole tokens per
    # workgroup, 3 the flat one); the cache is the front of a larger buffer whose two guard blocks must stay untouched
    announce(f"store slots past the cache, hkv {hkv}")
    rng = np.random.default_rng([hkv, 99])
    nb, bs, d, tokens = 6, 64, 128, 40
    buf_k = torch.full((nb + 2, bs, hkv, d), -3, dtype=torch.int16, device=dev).view(torch.bfloat16)
    buf_v = torch.full((nb + 2, bs, hkv, d), -4, dtype=torch.int16, device=dev).view(torch.bfloat16)
    kc, vc = buf_k[:nb], buf_v[:nb]
    k = torch.from_numpy(rng.integers(0, 1 << 16, size=(tokens, hkv, d), dtype=np.uint16).view(np.int16))
    v = torch.from_numpy(rng.integers(0, 1 << 16, size=(tokens, hkv, d), dtype=np.uint16).view(np.int16))
    k, v = k.to(dev).view(torch.bfloat16), v.to(dev).view(torch.bfloat16)
    slots_np = rng.permutation(nb * bs)[:tokens].astype(np.int32)
    slots_np[[1, 7, 20, 39]] = [nb * bs, nb * bs + 1, nb * bs + bs + 5, (nb + 2) * bs - 1]
    slots_np[3] = -1
    guard_k, guard_v = tensors.to_u16(buf_k[nb:]), tensors.to_u16(buf_v[nb:])
    kc0, vc0 = tensors.to_u16(kc), tensors.to_u16(vc)
    pa.pa_store_kvcache(k, v, kc, vc, torch.from_numpy(slots_np).to(dev))
    torch.cuda.synchronize()
    kref, vref = oracle.store_kvcache(tensors.to_u16(k), tensors.to_u16(v), slots_np, kc0, vc0)
    assert np.array_equal(tensors.to_u16(kc), kref)
    assert np.array_equal(tensors.to_u16(vc), vref)
    assert np.array_equal(tensors.to_u16(buf_k[nb:]), guard_k)
    assert np.array_equal(tensors.to_u16(buf_v[nb:]), guard_v)


def test_store_empty(dev):
    announce("store with zero tokens")
    kc = torch.zeros((2, 64, 1, 128), dtype=torch.bfloat16, device=dev)
    e = torch.zeros((0, 1, 128), dtype=torch.bfloat16, device=dev)
    pa.pa_store_kvcache(e, e, kc, kc, torch.zeros(0, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert int(kc.abs().sum()) == 0


@pytest.mark.parametrize("hkv,head_dim,tokens", [(1, 128, 37), (2, 64, 5), (3, 128, 29), (4, 128, 258), (8, 128, 1),
                                                 (8, 128, 513), (16, 128, 33), (6, 64, 17), (1, 8, 300)])
def test_store_head_layouts(dev, hkv, head_dim, tokens):
    """Both layouts of the store kernel: whole tokens per workgroup (K+V row a
    power of two of 16-byte vectors up to 256: hkv 1/2/4/8 at 128 dims, the
    8-element row) and the flat one (hkv 3, 6, 16); odd token counts, strided
    sources, padded slots."""
    announce(f"store hkv {hkv} head_dim {head_dim} tokens {tokens}")
    rng = np.random.default_rng([hkv, head_dim, tokens])
    nb, bs = 24, 32
    row = hkv * head_dim
    src = torch.from_numpy(rng.integers(0, 1 << 16, size=(tokens, 3 * row), dtype=np.uint16).view(np.int16)).to(dev)
    k = src[:, row:2 * row].view(torch.bfloat16).unflatten(1, (hkv, head_dim))
    v = src[:, 2 * row:].view(torch.bfloat16).unflatten(1, (hkv, head_dim))
    slots_np = rng.permutation(nb * bs)[:tokens].astype(np.int32)
    slots_np[rng.random(tokens) < 0.1] = -1
    slots = torch.from_numpy(slots_np).to(dev)
    kc = torch.full((nb, bs, hkv, head_dim), -1, dtype=torch.int16, device=dev).view(torch.bfloat16)
    vc = torch.full((nb, bs, hkv, head_dim), -2, dtype=torch.int16, device=dev).view(torch.bfloat16)
    kc0, vc0 = tensors.to_u16(kc), tensors.to_u16(vc)
    pa.pa_store_kvcache(k, v, kc, vc, slots)
    torch.cuda.synchronize()
    kref, vref = oracle.store_kvcache(tensors.to_u16(k), tensors.to_u16(v), slots_np, kc0, vc0)
    assert np.array_equal(tensors.to_u16(kc), kref)
    assert np.array_equal(tensors.to_u16(vc), vref)
