"""pa_decode on the GPU against the oracle (per-element tolerance)."""

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


def _run(wl, dev, seqs=None, split_waves=0, extra_check=None, scale=None):
    """store + decode on the GPU; the oracle repeats both on a host copy of the sampled sequences."""
    batch = tensors.materialize(wl, dev)
    seqs = list(range(wl.num_seqs)) if seqs is None else list(seqs)
    host = Compact(batch, seqs)  # pre-store contents
    k_new, v_new = tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new)
    q = tensors.to_u16(batch.q)
    slots = batch.slot_mapping.cpu().numpy()
    scale = 1.0 / math.sqrt(wl.head_dim) if scale is None else scale
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out = pa.pa_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables, batch.context_lens, scale,
                       wl.max_context_len, split_waves=split_waves)
    torch.cuda.synchronize()
    host.store(k_new, v_new, slots, wl.block_size)
    ref = oracle.decode(q[seqs], host.k, host.v, host.tables, wl.context_lens[seqs], scale)
    stats = assert_attention_close(out[seqs], ref, f"pa_decode {wl.name}")
    if extra_check:
        extra_check(batch, out)
    return stats


def test_decode_config1(dev):
    announce("decode config 1")
    wl = configs.config1()

    def one_token_is_v(batch, out):
        # the L = 1 sequence attends only to its just-stored token: out == v bit for bit
        g = wl.group
        for h in range(wl.num_q_heads):
            assert torch.equal(out[0, h].view(torch.int16), batch.v_new[0, h // g].view(torch.int16))

    _run(wl, dev, extra_check=one_token_is_v)


@pytest.mark.parametrize("seed", [2, 101, 102])
def test_decode_config2(dev, seed):
    announce(f"decode config 2 seed {seed}")
    _run(configs.config2(seed), dev)


@pytest.mark.parametrize("waves", [0, 1, 7, 300, 5000])
def test_decode_config2_splits(dev, waves):
    # 1 wave: every pair whole; 7..5000: pairs cut across 2 to many waves
    announce(f"decode config 2 split over {waves} waves")
    _run(configs.config2(), dev, split_waves=waves)


@pytest.mark.parametrize("group", [4, 8])
@pytest.mark.parametrize("waves", [0, 1, 7, 300, 5000])
def test_decode_matrix_core_splits(dev, group, waves):
    # the matrix-core split pass (G >= 4) over 64 sequences of config-2 lengths: 1 wave holds every pair whole,
    # 7..5000 waves cut pairs across 2 to many waves
    announce(f"decode G={group} split over {waves} waves")
    lens = np.random.default_rng([2, 0]).integers(100, 2048, size=64, endpoint=True)
    wl = configs.decode_workload(f"g{group}-64seq", lens, 8 * group, 8, 1024, 2)
    _run(wl, dev, split_waves=waves)


def test_decode_config5_sampled(dev):
    announce("decode config 5, sampled sequences")
    wl = configs.config5()
    lens = wl.context_lens
    order = np.argsort(lens)
    rng = np.random.default_rng(55)
    seqs = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2])] +
                      [int(x) for x in rng.choice(wl.num_seqs, 9, replace=False)]))
    _run(wl, dev, seqs=seqs)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("block_size", [64, 192, 256])
def test_decode_edge_lengths(dev, group, block_size):
    # empty context, one token, chunk, block and share boundaries (192: blocks that are not a power of two), a ragged tail
    lens = [0, 1, 2, 63, 64, 65, 191, 192, 193, 255, 256, 257, 383, 384, 385, 511, 512, 513, 1000, 1537]
    announce(f"decode edge lengths G={group} bs={block_size}")
    hkv = 2
    wl = configs.decode_workload("edge", lens, hkv * group, hkv, 128, seed=9, block_size=block_size)
    for waves in (0, 3, 64):
        _run(wl, dev, split_waves=waves)


@pytest.mark.parametrize("group", [2, 4])
@pytest.mark.parametrize("waves", [0, 77, 3000])
def test_decode_many_sequences(dev, group, waves):
    # 1500 short contexts (empty ones among them): the length scans of the split and finalize kernels walk six
    # 256-sequence windows, and pairs are cut across every window boundary
    announce(f"decode 1500 sequences G={group} waves={waves}")
    lens = np.random.default_rng(70 + group).integers(0, 300, size=1500)
    lens[::97] = 0
    hkv = 2
    wl = configs.decode_workload("many", lens, hkv * group, hkv, 2000, seed=41)
    rng = np.random.default_rng(5)
    seqs = sorted(set([0, 255, 256, 511, 512, 1023, 1024, 1499] + [int(x) for x in rng.choice(1500, 40, replace=False)]))
    _run(wl, dev, seqs=seqs, split_waves=waves)


def test_decode_zero_seqs(dev):
    announce("decode with zero sequences")
    kc = torch.zeros((1, 256, 8, 128), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((0, 16, 128), dtype=torch.bfloat16, device=dev)
    i = torch.zeros((0, 1), dtype=torch.int32, device=dev)
    out = pa.pa_decode(q, kc, kc, i, i[:, 0], 0.1, 0)
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 128)


def test_decode_identical_keys_gives_mean(dev):
    # every key equal -> uniform weights -> the mean of V (per kv head)
    announce("decode identical keys")
    wl = configs.decode_workload("ident", [300, 1], 4, 2, 4, seed=4)
    batch = tensors.materialize(wl, dev, fill_nan=False)
    key = batch.k_cache[0, 0].clone()
    batch.k_cache[:] = key
    batch.k_new[:] = key
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out = pa.pa_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables, batch.context_lens, 0.3, 300)
    torch.cuda.synchronize()
    v = tensors.to_u16(batch.v_cache)
    vf = oracle.bf16_to_f64(v)
    rows = [vf[wl.block_tables[0, p // 256], p % 256] for p in range(300)]
    mean = np.mean(rows, axis=0)  # [Hkv, D]
    want = np.stack([mean[h // 2] for h in range(4)])
    assert_attention_close(out[0], want, "identical keys")


def test_decode_block_permutation_invariant(dev):
    # moving a sequence's blocks elsewhere in the pool leaves the GPU result bit-identical
    announce("decode block permutation")
    wl = configs.decode_workload("perm", [700, 33, 1200], 16, 8, 32, seed=12)
    batch = tensors.materialize(wl, dev)
    pa.pa_store_kvcache(batch.k_new, batch.v_new, batch.k_cache, batch.v_cache, batch.slot_mapping)
    out1 = pa.pa_decode(batch.q, batch.k_cache, batch.v_cache, batch.block_tables, batch.context_lens, 0.088, 1200)
    sigma = torch.randperm(wl.num_blocks, generator=torch.Generator().manual_seed(3)).to(dev)
    kc2, vc2 = torch.empty_like(batch.k_cache), torch.empty_like(batch.v_cache)
    kc2[sigma], vc2[sigma] = batch.k_cache, batch.v_cache
    t = batch.block_tables.long()
    t2 = torch.where(t >= 0, sigma[t.clamp(min=0)], -1).to(torch.int32)
    out2 = pa.pa_decode(batch.q, kc2, vc2, t2, batch.context_lens, 0.088, 1200)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("scale", [0.0, -0.05])
def test_decode_nonpositive_scale(dev, scale):
    # scale 0 gives the mean of the context's values; a negative scale weights low scores most
    announce(f"decode scale {scale}")
    _run(configs.config1(), dev, scale=scale)
    _run(configs.config2(2), dev, seqs=range(0, 256, 17), split_waves=300, scale=scale)


@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_decode_pairs_cut_into_many_pieces(dev, group):
    # one long context over thousands of waves: each (sequence, kv head) pair is cut into hundreds of
    # pieces, which the finalize pass merges in batches of 64 and load rounds of 16 / 8 / 4 pieces
    announce(f"decode many pieces G={group}")
    wl = configs.decode_workload("pieces", [16384, 3, 700], 2 * group, 2, 72, seed=17)
    _run(wl, dev, split_waves=3000)


@pytest.mark.parametrize("group", [2, 4])
def test_decode_128k_context(dev, group):
    # one 131072-token context (512 blocks in the table) beside a short one: the vector (G = 2) and matrix-core
    # (G = 4) split passes cut each of its pairs into hundreds of pieces at the default split
    announce(f"decode 128k context G={group}")
    hkv = 2
    wl = configs.decode_workload("ctx-128k", [131072, 77], hkv * group, hkv, 520, seed=29)
    _run(wl, dev)
