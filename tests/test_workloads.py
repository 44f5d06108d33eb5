"""Workload generators: determinism, ranges, and the slot bookkeeping pinned to the oracle."""

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16, configs, tensors


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_slots_follow_oracle_definition(k):
    wl = configs.get(k)
    for slot, s, p in zip(wl.slot_mapping, wl.store_seq, wl.store_pos):
        assert slot == oracle.slot_of(wl.block_tables[s], int(p), wl.block_size)
    assert len(np.unique(wl.slot_mapping)) == len(wl.slot_mapping)
    assert wl.slot_mapping.min() >= 0 and wl.slot_mapping.max() < wl.num_blocks * wl.block_size


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_deterministic(k):
    a, b = configs.get(k), configs.get(k)
    assert np.array_equal(a.block_tables, b.block_tables) and np.array_equal(a.slot_mapping, b.slot_mapping)
    c = configs.get(k, seed=101)
    assert not np.array_equal(a.block_tables, c.block_tables)


def _used_blocks(wl):
    out = []
    for s, n in enumerate(wl.kv_lens()):
        out.extend(int(x) for x in wl.block_tables[s, :configs.blocks_for(n, wl.block_size)])
    return out


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_tables_disjoint(k):
    used = _used_blocks(configs.get(k))
    assert len(used) == len(set(used))


def test_config_shapes():
    c1 = configs.config1()
    assert list(c1.context_lens) == [1, 37, 256, 300] and c1.num_blocks == 16
    assert (c1.block_tables >= 0).sum() == 5
    c2 = configs.config2()
    assert c2.num_seqs == 256 and c2.context_lens.min() >= 100 and c2.context_lens.max() <= 2048
    c3 = configs.config3()
    n = np.diff(c3.cu_seqlens_q)
    assert n.sum() <= 16384 and n.min() >= 100 and n.max() <= 1024
    assert np.array_equal(c3.cu_seqlens_q, c3.cu_seqlens_k)
    c4 = configs.config4()
    m = np.diff(c4.cu_seqlens_q)
    assert c4.num_seqs == 32 and m.min() >= 128 and m.max() <= 512
    assert np.array_equal(np.diff(c4.cu_seqlens_k), m + 1024)
    assert all(np.array_equal(c4.block_tables[i, :4], c4.shared_prefix_blocks) for i in range(32))
    used = _used_blocks(c4)
    assert len(set(used)) == len(used) - 31 * 4  # only the prefix blocks repeat
    c5 = configs.config5()
    assert c5.num_blocks == 164794 and c5.num_q_heads == 32
    assert c5.context_lens.min() >= 256 and c5.context_lens.max() <= 32768


def test_admission_stops_at_first_overflow():
    assert configs.admitted_lengths([10, 20, 30, 5], 35) == [10, 20]
    assert configs.admitted_lengths([40], 35) == []


def test_bf16_encode_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 7
    x[:4] = [np.nan, np.inf, -np.inf, 3.0e38]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = bf16.encode(x)
    ok = ~np.isnan(x)
    assert np.array_equal(got[ok], ref[ok]) and got[0] == 0x7FC0
    # ties round to even: 1 + 2^-8 is halfway between two bf16 values
    assert bf16.encode(np.float32(1 + 2 ** -8)) == 0x3F80
    assert bf16.encode(np.float32(1 + 3 * 2 ** -8)) == 0x3F82


def test_materialize_cpu_layout():
    wl = configs.decode_workload("t", [1, 70, 5], 4, 2, 8, seed=3, block_size=64)
    b = tensors.materialize(wl, "cpu")
    kc = tensors.to_u16(b.k_cache)
    for s, n in enumerate(wl.context_lens):
        for p in range(wl.block_size * wl.block_tables.shape[1]):
            if p // 64 >= configs.blocks_for(n, 64):
                continue
            row = kc[wl.block_tables[s, p // 64], p % 64]
            if p < n - 1:
                assert not np.any(row == 0x7FC0)
            else:
                assert np.all(row == 0x7FC0)  # the new token's slot and the block tail
    assert b.k_new.stride(0) == (4 + 2 * 2) * 128 and b.q.shape == (3, 4, 128)
    assert list(b.slot_mapping.numpy()) == list(wl.slot_mapping)
