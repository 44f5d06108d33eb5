"""pa_store_decode_noalloc (the decode step with the library's static scratch, for callers that cannot
allocate) against pa_store_decode (caller workspace) through the C ABI: outputs and caches bit-identical
on two calls in a row, the second with a smaller input, and a third at another group size."""

import math

import pytest
import torch

import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401
from workloads import configs, tensors

pytestmark = pytest.mark.gpu


def _pair(wl, dev, split_waves=0):
    """Run both entry points on two copies of the same batch; return (out, caches) of each."""
    b = tensors.materialize(wl, dev)
    kc2, vc2 = b.k_cache.clone(), b.v_cache.clone()
    scale = 1.0 / math.sqrt(wl.head_dim)
    hq = wl.num_q_heads
    out_ref = pa.pa_store_decode(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                 scale, wl.max_context_len, split_waves=split_waves)
    out = torch.full((wl.num_seqs, hq, wl.head_dim), float("nan"), dtype=torch.bfloat16, device=dev)
    pa.pa_store_decode_noalloc(b.q, b.k_new, b.v_new, kc2, vc2, b.block_tables, b.context_lens, scale,
                               wl.max_context_len, out, split_waves=split_waves)
    torch.cuda.synchronize()
    return (out_ref, b.k_cache, b.v_cache), (out, kc2, vc2)


def _same(a, b, what):
    for x, y, name in zip(a, b, ("out", "k_cache", "v_cache")):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{what}: {name} differs"


def test_noalloc_matches_store_decode_two_calls(dev):
    # first call: the 256-sequence decode batch (the scratch's default split of 2048 waves, many cut pairs);
    # second call: the 4-sequence tiny batch, smaller, on the scratch the first call left behind
    announce("no-alloc decode: 256-seq batch then 4-seq batch")
    ref, got = _pair(configs.config2(), dev)
    _same(ref, got, "decode batch")
    ref, got = _pair(configs.config1(), dev)
    _same(ref, got, "tiny batch after the decode batch")


@pytest.mark.parametrize("group", [4, 8])
def test_noalloc_other_groups(dev, group):
    # larger groups use more of the scratch per wave: 300 waves and the default split
    announce(f"no-alloc decode G={group}")
    lens = [0, 1, 17, 300, 1537, 4000, 255, 256, 257]
    wl = configs.decode_workload("noalloc", lens, 2 * group, 2, 64, seed=41)
    for waves in (300, 0):
        ref, got = _pair(wl, dev, split_waves=waves)
        _same(ref, got, f"G={group} waves={waves}")


def test_noalloc_refuses_a_split_beyond_the_scratch(dev):
    announce("no-alloc decode: split beyond the static scratch")
    wl = configs.decode_workload("noalloc-big", [3000] * 8, 64, 8, 128, seed=42)
    b = tensors.materialize(wl, dev)
    out = torch.empty((8, 64, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(pa.PAError, match="static scratch"):
        pa.pa_store_decode_noalloc(b.q, b.k_new, b.v_new, b.k_cache, b.v_cache, b.block_tables, b.context_lens,
                                   0.088, wl.max_context_len, out, split_waves=2049)
