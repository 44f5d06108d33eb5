"""pa_store_prefill_varlen (the new tokens' store fused into varlen prefill) against the unfused pair
pa_store_kvcache + pa_prefill_varlen run on copies of the same batch: the caches byte for byte and the
outputs bit for bit, and the outputs against the oracle (store, then prefill).

Cases: the packed varlen workload (every key new), the prefix-cached workload (a shared 1024-token prefix
read through the table, the new tokens from k_new), a chunked prefill whose cached part ends mid-tile
(tiles that take their first rows from the cache and the rest from k_new) for G = 1, 2, 4, 8, causal and
not, 64- and 256-token blocks, and padded or out-of-pool slots (nothing stored)."""

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


def _bits(t):
    return t.view(torch.int16)


def _i32(a, dev):
    return torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(dev)


def _compare(q, k_new, v_new, k_cache, v_cache, slots, cu_q, cu_k, max_q, max_k, scale, causal, table, what):
    """Fused on the given caches, unfused on copies; both must agree exactly. Returns the fused output."""
    kc2, vc2 = k_cache.clone(), v_cache.clone()
    out = pa.pa_store_prefill_varlen(q, k_new, v_new, k_cache, v_cache, slots, cu_q, cu_k, max_q, max_k, scale,
                                     causal=causal, block_table=table)
    pa.pa_store_kvcache(k_new, v_new, kc2, vc2, slots)
    if table is None:
        ref = pa.pa_prefill_varlen(q, k_new, v_new, cu_q, cu_k, max_q, max_k, scale, causal=causal)
    else:
        # with a block table the fused call runs 64-key tiles; the unfused call is given a key bound above
        # 1024 (and a table padded with never-read entries to cover it) so that it runs them too
        mk = max(max_k, 1025)
        bs = k_cache.shape[1]
        pad = -(-mk // bs) - table.shape[1]
        wide = table if pad <= 0 else torch.cat(
            [table, torch.full((table.shape[0], pad), -1, dtype=table.dtype, device=table.device)], 1).contiguous()
        ref = pa.pa_prefill_varlen(q, kc2, vc2, cu_q, cu_k, max_q, mk, scale, causal=causal, block_table=wide)
    torch.cuda.synchronize()
    assert torch.equal(_bits(k_cache), _bits(kc2)) and torch.equal(_bits(v_cache), _bits(vc2)), f"{what}: caches"
    assert torch.equal(_bits(out), _bits(ref)), f"{what}: output differs from the unfused pair"
    return out


@pytest.mark.parametrize("max_k", [None, 4096])
def test_fused_varlen_workload(dev, max_k):
    announce(f"fused store + prefill, varlen workload, max_k {max_k}")
    wl = configs.config3()
    b = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    mk = wl.max_seqlen_k if max_k is None else max_k
    out = _compare(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.slot_mapping, b.cu_seqlens_q, b.cu_seqlens_k,
                   wl.max_seqlen_q, mk, scale, True, None, wl.name)
    ref = oracle.prefill_varlen(tensors.to_u16(b.q), tensors.to_u16(b.k_new), tensors.to_u16(b.v_new),
                                wl.cu_seqlens_q, wl.cu_seqlens_k, scale)
    assert_attention_close(out, ref, f"pa_store_prefill_varlen {wl.name}")


def test_fused_prefix_workload(dev):
    announce("fused store + prefill, prefix-cached workload")
    wl = configs.config4()
    b = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    host = Compact(b, range(wl.num_seqs))  # pre-store contents
    k_new, v_new = tensors.to_u16(b.k_new), tensors.to_u16(b.v_new)
    slots = b.slot_mapping.cpu().numpy()
    out = _compare(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.slot_mapping, b.cu_seqlens_q, b.cu_seqlens_k,
                   wl.max_seqlen_q, wl.max_seqlen_k, scale, True, b.block_tables, wl.name)
    host.store(k_new, v_new, slots, wl.block_size)
    ref = oracle.prefill_varlen(tensors.to_u16(b.q), host.k, host.v, wl.cu_seqlens_q, wl.cu_seqlens_k, scale,
                                block_table=host.tables)
    assert_attention_close(out, ref, f"pa_store_prefill_varlen {wl.name}")


@pytest.mark.parametrize("block_size", [64, 192, 256])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_fused_chunked_prefill_cached_part_ends_mid_tile(dev, group, causal, block_size):
    # each sequence already holds its first c tokens (stored earlier, in its own blocks); the rest are
    # new: with c = 37, 100, 63, 250 the first tile that needs new tokens also needs cached rows
    announce(f"fused store + prefill, chunked, G={group} causal={causal} bs={block_size}")
    lens = np.array([300, 180, 64, 700, 129])
    cached = np.array([37, 100, 0, 250, 63])
    hkv = 2
    nb = int(sum(-(-int(n) // block_size) for n in lens)) + 3
    wl = configs.prefill_workload("chunked", lens, 0, hkv * group, hkv, nb, seed=31, block_size=block_size)
    b = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    starts = wl.cu_seqlens_q[:-1]
    old = np.concatenate([np.arange(s, s + c) for s, c in zip(starts, cached)])
    new = np.concatenate([np.arange(s + c, s + n) for s, c, n in zip(starts, cached, lens)])
    old_t, new_t = torch.as_tensor(old, device=dev), torch.as_tensor(new, device=dev)
    pa.pa_store_kvcache(b.k_new[old_t], b.v_new[old_t], b.k_cache, b.v_cache, b.slot_mapping[old_t])
    host = Compact(b, range(wl.num_seqs))  # the cached parts in place
    q, k_new, v_new = b.q[new_t].contiguous(), b.k_new[new_t].contiguous(), b.v_new[new_t].contiguous()
    slots = b.slot_mapping[new_t].contiguous()
    cu_q = np.concatenate([[0], np.cumsum(lens - cached)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = _compare(q, k_new, v_new, b.k_cache, b.v_cache, slots, _i32(cu_q, dev), _i32(cu_k, dev),
                   int((lens - cached).max()), int(lens.max()), scale, causal, b.block_tables, "chunked")
    host.store(tensors.to_u16(k_new), tensors.to_u16(v_new), slots.cpu().numpy(), wl.block_size)
    ref = oracle.prefill_varlen(tensors.to_u16(q), host.k, host.v, cu_q, cu_k, scale, causal=causal,
                                block_table=host.tables)
    assert_attention_close(out, ref, "pa_store_prefill_varlen chunked")


def test_fused_padded_and_out_of_pool_slots_store_nothing(dev):
    # packed: slots -1 and past the pool are skipped; attention still sees every key (packed)
    announce("fused store + prefill, padded and out-of-pool slots")
    wl = configs.prefill_workload("pad", [5, 0, 70, 33], 0, 4, 2, 16, seed=23)
    b = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    slots = b.slot_mapping.clone()
    slots[3] = -1
    slots[10] = wl.num_blocks * wl.block_size + 5  # past the pool
    kc0, vc0 = b.k_cache.clone(), b.v_cache.clone()
    out = pa.pa_store_prefill_varlen(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, slots, b.cu_seqlens_q,
                                     b.cu_seqlens_k, wl.max_seqlen_q, wl.max_seqlen_k, scale)
    ref = pa.pa_prefill_varlen(b.q, b.k_new, b.v_new, b.cu_seqlens_q, b.cu_seqlens_k, wl.max_seqlen_q,
                               wl.max_seqlen_k, scale)
    stored = slots.clone()
    stored[10] = -1  # what an unfused store may be given: the same skips
    pa.pa_store_kvcache(b.k_new, b.v_new, kc0, vc0, stored)
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref))
    assert torch.equal(_bits(b.k_cache), _bits(kc0)) and torch.equal(_bits(b.v_cache), _bits(vc0))
