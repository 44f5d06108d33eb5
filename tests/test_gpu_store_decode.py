"""pa_store_decode (store of the new tokens + decode in one launch) on the GPU.

Against the two separate calls on a copy of the same batch: the caches must be
bit-identical afterwards (the fused call writes each sequence's new row at
position L - 1 through its block table; the workload's slot_mapping names the
same slot), and the outputs bit-identical at the same work split (the fused
call reads the row it stored, so every product and sum is the same); and
against the oracle's store + decode within the attention tolerance.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401
from tests.parity import Compact, assert_attention_close
from workloads import configs, tensors

pytestmark = pytest.mark.gpu


def _run(wl, dev, split_waves=0, oracle_seqs=None):
    batch = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    kc2, vc2 = batch.k_cache.clone(), batch.v_cache.clone()
    seqs = list(range(wl.num_seqs)) if oracle_seqs is None else list(oracle_seqs)
    host = Compact(batch, seqs)  # pre-store contents
    # separate calls on the copies
    pa.pa_store_kvcache(batch.k_new, batch.v_new, kc2, vc2, batch.slot_mapping)
    ref_out = pa.pa_decode(batch.q, kc2, vc2, batch.block_tables, batch.context_lens, scale, wl.max_context_len,
                           split_waves=split_waves)
    # the fused call on the originals
    out = pa.pa_store_decode(batch.q, batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.block_tables,
                             batch.context_lens, scale, wl.max_context_len, split_waves=split_waves)
    torch.cuda.synchronize()
    assert torch.equal(batch.k_cache.view(torch.int16), kc2.view(torch.int16)), "K cache differs"
    assert torch.equal(batch.v_cache.view(torch.int16), vc2.view(torch.int16)), "V cache differs"
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), "output differs from store + decode"
    host.store(tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new), batch.slot_mapping.cpu().numpy(),
               wl.block_size)
    ref = oracle.decode(tensors.to_u16(batch.q)[seqs], host.k, host.v, host.tables, wl.context_lens[seqs], scale)
    assert_attention_close(out[seqs], ref, f"pa_store_decode {wl.name}")


def test_store_decode_config1(dev):
    announce("store+decode config 1")
    _run(configs.config1(), dev)


@pytest.mark.parametrize("split_waves", [0, 300])
def test_store_decode_config2(dev, split_waves):
    announce(f"store+decode config 2 split {split_waves}")
    _run(configs.config2(), dev, split_waves=split_waves, oracle_seqs=range(0, 256, 17))


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("block_size", [64, 192, 256])
def test_store_decode_edge_lengths(dev, group, block_size):
    # empty context (nothing stored), one token (the stored row alone), chunk and block edges
    lens = [0, 1, 2, 63, 64, 65, 191, 192, 193, 255, 256, 257, 383, 384, 385, 511, 512, 513, 1000, 1537]
    announce(f"store+decode edge lengths G={group} bs={block_size}")
    hkv = 2
    wl = configs.decode_workload("edge", lens, hkv * group, hkv, 128, seed=19, block_size=block_size)
    for waves in (0, 3, 64):
        _run(wl, dev, split_waves=waves)


def test_store_decode_one_token_returns_v(dev):
    # L = 1: the output is the row just stored, bit for bit in bf16
    announce("store+decode one-token contexts")
    wl = configs.decode_workload("one", [1, 1, 1], 16, 8, 16, seed=29)
    batch = tensors.materialize(wl, dev)
    out = pa.pa_store_decode(batch.q, batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.block_tables,
                             batch.context_lens, 0.088, 1)
    torch.cuda.synchronize()
    want = batch.v_new.repeat_interleave(2, dim=1)  # q head h reads kv head h // 2
    assert torch.equal(out.view(torch.int16), want.contiguous().view(torch.int16))
