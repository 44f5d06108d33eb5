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


def test_store_empty(dev):
    announce("store with zero tokens")
    kc = torch.zeros((2, 64, 1, 128), dtype=torch.bfloat16, device=dev)
    e = torch.zeros((0, 1, 128), dtype=torch.bfloat16, device=dev)
    pa.pa_store_kvcache(e, e, kc, kc, torch.zeros(0, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    assert int(kc.abs().sum()) == 0
