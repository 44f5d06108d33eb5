"""pa_prefill_varlen on the GPU against the oracle (per-element tolerance)."""

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


def _cover(table, max_k: int, block_size: int):
    """The block table padded with never-read -1 columns until a row covers max_k keys (the library
    rejects a max_seqlen_k its table cannot address)."""
    need = -(-max_k // block_size) - table.shape[1]
    if need <= 0:
        return table
    pad = torch.full((table.shape[0], need), -1, dtype=table.dtype, device=table.device)
    return torch.cat([table, pad], dim=1).contiguous()


def _packed(wl, dev, causal=True, check_table_path=True, max_k=None, scale=None):
    """Prefill over packed q/k/v; the same keys read back through the cache must give identical bits.

    max_k overrides the max_seqlen_k hint, which only picks the key tile (1 -> 32 keys, 4096 -> 64 keys).
    scale defaults to 1/sqrt(head_dim).
    """
    mk = wl.max_seqlen_k if max_k is None else max_k
    batch = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim) if scale is None else scale
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out = pa.pa_prefill_varlen(batch.q, batch.k_new, batch.v_new, batch.cu_seqlens_q, batch.cu_seqlens_k,
                               wl.max_seqlen_q, mk, scale, causal=causal)
    out_t = None
    if check_table_path:
        out_t = pa.pa_prefill_varlen(batch.q, batch.k_cache, batch.v_cache, batch.cu_seqlens_q, batch.cu_seqlens_k,
                                     wl.max_seqlen_q, mk, scale, causal=causal,
                                     block_table=_cover(batch.block_tables, mk, wl.block_size))
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(tensors.to_u16(batch.q), tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new),
                                wl.cu_seqlens_q, wl.cu_seqlens_k, scale, causal=causal)
    stats = assert_attention_close(out, ref, f"pa_prefill_varlen packed {wl.name}")
    if out_t is not None:
        assert torch.equal(out.view(torch.int16), out_t.view(torch.int16)), "table path differs from packed path"
    return stats


def _table(wl, dev, causal=True, max_k=None):
    """store the new tokens, then prefill through the block table (prefix blocks shared)."""
    mk = wl.max_seqlen_k if max_k is None else max_k
    batch = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    host = Compact(batch, range(wl.num_seqs))  # pre-store contents
    k_new, v_new = tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new)
    slots = batch.slot_mapping.cpu().numpy()
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out = pa.pa_prefill_varlen(batch.q, batch.k_cache, batch.v_cache, batch.cu_seqlens_q, batch.cu_seqlens_k,
                               wl.max_seqlen_q, mk, scale, causal=causal,
                               block_table=_cover(batch.block_tables, mk, wl.block_size))
    torch.cuda.synchronize()
    host.store(k_new, v_new, slots, wl.block_size)
    ref = oracle.prefill_varlen(tensors.to_u16(batch.q), host.k, host.v, wl.cu_seqlens_q, wl.cu_seqlens_k, scale,
                                causal=causal, block_table=host.tables)
    return assert_attention_close(out, ref, f"pa_prefill_varlen table {wl.name}")


@pytest.mark.parametrize("seed,max_k", [(3, None), (101, None), (3, 4096)])
def test_prefill_config3(dev, seed, max_k):
    announce(f"prefill config 3 seed {seed} max_k {max_k}")
    _packed(configs.config3(seed), dev, max_k=max_k)


@pytest.mark.parametrize("seed,max_k", [(4, None), (102, None), (4, 1)])
def test_prefill_config4(dev, seed, max_k):
    announce(f"prefill config 4 seed {seed} max_k {max_k}")
    _table(configs.config4(seed), dev, max_k=max_k)


@pytest.mark.parametrize("max_k", [1, 4096])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_ragged_small(dev, group, causal, max_k):
    # lengths around tile edges (16, 32, 64, 128/G positions) and single-token sequences
    lens = [1, 2, 15, 16, 17, 31, 33, 63, 64, 65, 127, 129, 300]
    announce(f"prefill ragged G={group} causal={causal} max_k={max_k}")
    wl = configs.prefill_workload("ragged", lens, 0, 2 * group, 2, 64, seed=21)
    _packed(wl, dev, causal=causal, max_k=max_k)


@pytest.mark.parametrize("max_k", [1, 4096])
@pytest.mark.parametrize("block_size", [64, 192, 256])
@pytest.mark.parametrize("group", [2, 4])
def test_prefill_prefix_small(dev, block_size, group, max_k):
    # fewer queries than keys: queries are the last positions; prefix blocks shared (the prefix is the
    # whole blocks covering 256 tokens: 384 at block size 192)
    announce(f"prefill prefix bs={block_size} G={group} max_k={max_k}")
    prefix = -(-256 // block_size) * block_size
    wl = configs.prefill_workload("prefix", [1, 5, 64, 100, 200], prefix, 2 * group, 2, 64, seed=22,
                                  block_size=block_size)
    _table(wl, dev, causal=True, max_k=max_k)
    _table(wl, dev, causal=False, max_k=max_k)


@pytest.mark.parametrize("max_k", [1, 4096])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_prefill_nonpositive_scale(dev, group, scale, max_k):
    # a scale <= 0 takes the kernel's other softmax form (scores scaled before the running maximum);
    # scale 0 gives the mean of the visible values
    announce(f"prefill scale {scale} G={group} max_k={max_k}")
    wl = configs.prefill_workload("scale", [1, 17, 64, 65, 200], 0, 2 * group, 2, 64, seed=24)
    _packed(wl, dev, causal=True, max_k=max_k, scale=scale)


@pytest.mark.parametrize("max_k", [1, 8192])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_table_past_64_blocks(dev, causal, max_k):
    # 64-token blocks and a 4608-token cached prefix: the tables run past 64 entries, so the kernel
    # reloads its cached table entries mid-sequence
    announce(f"prefill table > 64 blocks causal={causal} max_k={max_k}")
    wl = configs.prefill_workload("long-table", [300, 37], 4608, 4, 2, 96, seed=25, block_size=64)
    assert wl.block_tables.shape[1] > 64
    _table(wl, dev, causal=causal, max_k=max_k)


def test_prefill_empty_sequence_in_batch(dev):
    announce("prefill with an empty sequence in the batch")
    wl = configs.prefill_workload("empty", [5, 0, 70], 0, 4, 2, 16, seed=23)
    _packed(wl, dev)


def test_prefill_last_row_equals_decode(dev):
    # the last query row of each sequence sees the same keys as a decode over that sequence
    announce("prefill last row vs decode")
    lens = [1, 77, 256, 300]
    wl = configs.prefill_workload("lastrow", lens, 0, 16, 8, 16, seed=24)
    batch = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(128)
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out = pa.pa_prefill_varlen(batch.q, batch.k_cache, batch.v_cache, batch.cu_seqlens_q, batch.cu_seqlens_k,
                               wl.max_seqlen_q, wl.max_seqlen_k, scale, block_table=batch.block_tables)
    last = torch.tensor(wl.cu_seqlens_q[1:] - 1, dtype=torch.int64, device=dev)
    q_last = batch.q[last].contiguous()
    lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)
    dec = pa.pa_decode(q_last, batch.k_cache, batch.v_cache, batch.block_tables, lens_t, scale, max(lens))
    torch.cuda.synchronize()
    # both are within tolerance of the same oracle rows; they use different arithmetic (MFMA vs dot2)
    ref = oracle.prefill_varlen(tensors.to_u16(batch.q), tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new),
                                wl.cu_seqlens_q, wl.cu_seqlens_k, scale)[wl.cu_seqlens_q[1:] - 1]
    assert_attention_close(out[last], ref, "prefill last rows")
    assert_attention_close(dec, ref, "decode of the same rows")


@pytest.mark.parametrize("max_k", [None, 1000])
def test_prefill_one_sequence_fills_the_batch(dev, max_k):
    # the largest prefill one 16384-token batch holds: one sequence of 16384 tokens (256 query tiles, up to 16384
    # keys a row), at 64-key tiles (default) and 32-key tiles (the hint 1000), packed and through a 256-entry table
    # of 64-token blocks (the kernel reloads its 64 held entries three times); sampled rows against the oracle
    n, bs = 16384, 64
    announce(f"prefill one {n}-token sequence max_k {max_k}")
    wl = configs.prefill_workload("one-seq-16k", [n], 0, 16, 8, n // bs + 8, seed=23, block_size=bs)
    batch = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(wl.head_dim)
    mk = wl.max_seqlen_k if max_k is None else max_k
    host = Compact(batch, [0])  # pre-store contents
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out = pa.pa_prefill_varlen(batch.q, batch.k_new, batch.v_new, batch.cu_seqlens_q, batch.cu_seqlens_k,
                               wl.max_seqlen_q, mk, scale)
    out_t = pa.pa_prefill_varlen(batch.q, batch.k_cache, batch.v_cache, batch.cu_seqlens_q, batch.cu_seqlens_k,
                                 wl.max_seqlen_q, mk, scale, block_table=_cover(batch.block_tables, mk, bs))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_t.view(torch.int16)), "table path differs from packed path"
    host.store(tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new), batch.slot_mapping.cpu().numpy(), bs)
    rng = np.random.default_rng(24)
    rows = sorted(set([0, 1, 2, 63, 64, 65, 127, 128, 1023, 1024, 4095, 4096, 8191, 8192, 16382, 16383] +
                      [int(x) for x in rng.choice(n, 24, replace=False)]))
    # row p of the sequence is the one query of a sequence of p + 1 keys read through the same table
    cu_q = np.arange(len(rows) + 1, dtype=np.int64)
    cu_k = np.concatenate([[0], np.cumsum(np.array(rows, dtype=np.int64) + 1)])
    ref = oracle.prefill_varlen(tensors.to_u16(batch.q)[rows], host.k, host.v, cu_q, cu_k, scale, causal=True,
                                block_table=np.repeat(host.tables[:1], len(rows), axis=0))
    assert_attention_close(out[rows], ref, f"pa_prefill_varlen packed one-seq-16k max_k {max_k}")
