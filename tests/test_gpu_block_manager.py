"""The C++ block manager's metadata driving the GPU kernels: prefix reuse end to end.

Eight sequences share a 512-token prompt prefix. The manager gives the first
sequence fresh blocks and the other seven its two prefix blocks (ref count 8);
only the computed tokens are stored; prefill through the manager's block
table must equal the oracle's prefill over each sequence's full K/V; then one
decode step with the manager's decode metadata must equal the oracle's decode.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_heads_amd as pa
from paged_kv_cache_heads_amd.blocks import BlockManager
from tests.gpu_common import announce, dev  # noqa: F401
from tests.parity import assert_attention_close
from workloads.bf16 import normal

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS, NB = 16, 8, 128, 256, 64


def _dev(a, dev):
    return torch.as_tensor(np.ascontiguousarray(a)).to(dev)


def _bf16(bits, dev):
    return _dev(bits.view(np.int16), dev).view(torch.bfloat16)


def test_prefix_reuse_prefill_then_decode(dev):
    announce("block manager -> store + prefill + decode")
    rng = np.random.default_rng(41)
    prefix = rng.integers(0, 32000, 512).tolist()
    tails = [300, 50, 1, 255, 256, 257, 100, 7]
    bm = BlockManager(NB, BS, order=rng.permutation(NB))
    cached = [bm.allocate(i, prefix + rng.integers(0, 32000, t).tolist()) for i, t in enumerate(tails)]
    assert cached == [0] + [512] * 7
    shared = bm.table(0)[:2]
    assert all(bm.table(i)[:2] == shared for i in range(8)) and bm.ref(shared[0]) == 8
    ids = list(range(8))
    width = 4
    bt, cq, ck, slots = bm.prefill_metadata(ids, cached, width)
    tq = int(cq[-1])
    assert tq == 512 + sum(tails)

    # K/V/q of the computed tokens (sequence 0 computes the prefix for everyone)
    k_new, v_new = normal(rng, (tq, HKV, D)), normal(rng, (tq, HKV, D))
    q = normal(rng, (tq, HQ, D))
    k_cache = torch.zeros((NB, BS, HKV, D), dtype=torch.bfloat16, device=dev)
    k_cache.view(torch.int16).fill_(0x7FC0)  # unwritten rows: NaN
    v_cache = k_cache.clone()
    kn, vn, qd = _bf16(k_new, dev), _bf16(v_new, dev), _bf16(q, dev)
    pa.pa_store_kvcache(kn, vn, k_cache, v_cache, _dev(slots, dev))
    scale = 1.0 / math.sqrt(D)
    out = pa.pa_prefill_varlen(qd, k_cache, v_cache, _dev(cq, dev), _dev(ck, dev), int(np.diff(cq).max()),
                               int(np.diff(ck).max()), scale, block_table=_dev(bt, dev))
    torch.cuda.synchronize()

    # oracle: each sequence's full K/V = the shared prefix rows (computed by sequence 0) + its own rows
    full_k, full_v = [], []
    for i in ids:
        own = slice(int(cq[i]), int(cq[i + 1]))
        if i == 0:
            full_k.append(k_new[own]), full_v.append(v_new[own])
        else:
            full_k.append(np.concatenate([k_new[:512], k_new[own]]))
            full_v.append(np.concatenate([v_new[:512], v_new[own]]))
    ref = oracle.prefill_varlen(q, np.concatenate(full_k), np.concatenate(full_v), cq, ck, scale)
    assert_attention_close(out, ref, "prefill through the manager's tables")

    # one decode step: the manager appends a token to every sequence and builds the metadata
    for i in ids:
        bm.append(i, 1)
    bt2, cl, slot2 = bm.decode_metadata(ids, width)
    k1, v1, q1 = normal(rng, (8, HKV, D)), normal(rng, (8, HKV, D)), normal(rng, (8, HQ, D))
    pa.pa_store_kvcache(_bf16(k1, dev), _bf16(v1, dev), k_cache, v_cache, _dev(slot2, dev))
    dec = pa.pa_decode(_bf16(q1, dev), k_cache, v_cache, _dev(bt2, dev), _dev(cl, dev), scale, int(cl.max()))
    torch.cuda.synchronize()
    refs = []
    for i in ids:
        kk = np.concatenate([full_k[i], k1[i:i + 1]])
        vv = np.concatenate([full_v[i], v1[i:i + 1]])
        n = len(kk)
        refs.append(oracle.prefill_varlen(q1[i:i + 1], kk, vv, np.array([0, 1]), np.array([0, n]), scale)[0])
    assert_attention_close(dec, np.stack(refs), "decode through the manager's tables")
