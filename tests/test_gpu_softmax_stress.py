"""Online-softmax stress: scores that grow (or fall) along the keys, for prefill and decode.

With k_t = beta * t * u + noise and q = +-u + noise (u the all-ones vector),
the score of key t is about +-beta * sqrt(D) * t: rising by about 1.5 per key
for the heads with +u, so the running row maximum moves on every key tile
(the lazy rescale fires every tile, and in decode every chunk) and the
softmax is dominated by the last visible keys, which also makes an
off-by-one in the causal or sequence-end mask show up as a large error; the
heads with -u see falling scores (the maximum stays on the first tile). Both
kinds of head share waves, so a rescale decided for one row set must leave
the other correct. Checked against the fp64 oracle with the usual tolerance.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401
from tests.parity import assert_attention_close
from workloads.bf16 import encode

pytestmark = pytest.mark.gpu

D = 128
BETA = 0.13


def _bits_to_dev(bits, dev):
    return torch.as_tensor(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def _queries(rng, n, hq):
    sign = np.where(np.arange(hq) % 2 == 0, 1.0, -1.0)[None, :, None]
    return encode(sign + 0.3 * rng.standard_normal((n, hq, D)))


def _keys(rng, pos, hkv):
    return encode(BETA * np.asarray(pos, np.float64)[:, None, None] + 0.3 * rng.standard_normal((len(pos), hkv, D)))


@pytest.mark.parametrize("max_k", [1, 4096])
@pytest.mark.parametrize("group", [2, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_growing_scores(dev, causal, group, max_k):
    announce(f"prefill growing scores causal={causal} G={group} max_k={max_k}")
    rng = np.random.default_rng(60 + group)
    hkv, hq = 2, 2 * group
    lens = [40, 300, 700]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pos = np.concatenate([np.arange(n) for n in lens])
    q, k = _queries(rng, int(cu[-1]), hq), _keys(rng, pos, hkv)
    v = encode(rng.standard_normal((int(cu[-1]), hkv, D)))
    cu_t = torch.as_tensor(cu).to(dev)
    scale = 1.0 / math.sqrt(D)
    out = pa.pa_prefill_varlen(_bits_to_dev(q, dev), _bits_to_dev(k, dev), _bits_to_dev(v, dev), cu_t, cu_t,
                               max(lens), max(lens) if max_k is None else max_k, scale, causal=causal)
    torch.cuda.synchronize()
    ref = oracle.prefill_varlen(q, k, v, cu, cu, scale, causal=causal)
    assert_attention_close(out, ref, "prefill, growing scores")


@pytest.mark.parametrize("split_waves", [0, 7, 300])
@pytest.mark.parametrize("group", [2, 4])
def test_decode_growing_scores(dev, group, split_waves):
    announce(f"decode growing scores G={group} split={split_waves}")
    rng = np.random.default_rng(70 + group)
    hkv, hq, bs, nb = 2, 2 * group, 256, 40
    lens = np.array([1, 37, 300, 1500, 2048, 511], dtype=np.int32)
    width = 8
    perm = rng.permutation(nb)
    tables = np.full((len(lens), width), -1, dtype=np.int32)
    k_cache = np.full((nb, bs, hkv, D), 0x7FC0, dtype=np.uint16)  # unwritten rows: NaN
    v_cache = k_cache.copy()
    nxt = 0
    for b, n in enumerate(lens):
        nblk = -(-int(n) // bs)
        tables[b, :nblk] = perm[nxt:nxt + nblk]
        nxt += nblk
        kb, vb = _keys(rng, np.arange(n), hkv), encode(rng.standard_normal((int(n), hkv, D)))
        for t in range(int(n)):
            k_cache[tables[b, t // bs], t % bs] = kb[t]
            v_cache[tables[b, t // bs], t % bs] = vb[t]
    q = _queries(rng, len(lens), hq)
    scale = 1.0 / math.sqrt(D)
    out = pa.pa_decode(_bits_to_dev(q, dev), _bits_to_dev(k_cache, dev), _bits_to_dev(v_cache, dev),
                       torch.as_tensor(tables).to(dev), torch.as_tensor(lens).to(dev), scale, int(lens.max()),
                       split_waves=split_waves)
    torch.cuda.synchronize()
    ref = oracle.decode(q, k_cache, v_cache, tables, lens, scale)
    assert_attention_close(out, ref, "decode, growing scores")
