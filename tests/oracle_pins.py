"""Checks that pin the fp64 oracle to facts other than itself.

Each ``check_*`` takes an oracle module (the real one, or a mutant built by
``test_oracle_mutants.py``) and raises ``AssertionError`` if the oracle breaks
the fact. The facts are: hand-worked golden examples (``tests/golden``),
closed forms, exact invariants of the definition, a pure-Python brute force
and ``torch.nn.functional.scaled_dot_product_attention`` in fp64.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

from workloads.bf16 import encode

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _scale(expr):
    return {"ln2": math.log(2.0), "1/sqrt(4)": 0.5}[expr]


def _cache(arr, hkv, d):
    """JSON cache [NB][bs][Hkv][D] with null rows -> bf16 NaN rows."""
    out = np.full((len(arr), len(arr[0]), hkv, d), np.nan)
    for b, blk in enumerate(arr):
        for r, row in enumerate(blk):
            for h, vec in enumerate(row):
                if vec is not None:
                    out[b, r, h] = vec
    return encode(out)


def _rand(rng, shape):
    return encode(rng.standard_normal(shape))


def _f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _paged_case(rng, lengths, hkv, d, block_size, perm=None, fill_nan=True):
    """Random K/V for sequences of the given lengths, placed in a shuffled pool.

    Returns (k_cache, v_cache, block_tables, packed_k, packed_v). Unused rows
    hold bf16 NaN so that any read of them shows up in the result.
    """
    need = [max(1, -(-n // block_size)) for n in lengths]
    nb = sum(need) + 2
    if perm is None:
        perm = rng.permutation(nb)
    width = max(need)
    tables = np.full((len(lengths), width), -1, dtype=np.int32)
    kc = np.full((nb, block_size, hkv, d), 0x7FC0 if fill_nan else 0, dtype=np.uint16)
    vc = kc.copy()
    packed_k, packed_v = [], []
    nxt = 0
    for i, n in enumerate(lengths):
        blocks = perm[nxt:nxt + need[i]]
        nxt += need[i]
        tables[i, :len(blocks)] = blocks
        ki = _rand(rng, (n, hkv, d))
        vi = _rand(rng, (n, hkv, d))
        for p in range(n):
            kc[blocks[p // block_size], p % block_size] = ki[p]
            vc[blocks[p // block_size], p % block_size] = vi[p]
        packed_k.append(ki)
        packed_v.append(vi)
    return kc, vc, tables, packed_k, packed_v


# --------------------------------------------------------------------------- golden


def check_bf16_widen(orc):
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x8000, 0x7F80, 0xFF80, 0x4049, 0x0080], dtype=np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, -0.0, math.inf, -math.inf, 3.140625, 2.0 ** -126]
    got = orc.bf16_to_f64(bits)
    assert list(got) == want, got
    assert np.isnan(orc.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])
    rnd = np.random.default_rng(7).integers(0, 1 << 16, 4096).astype(np.uint16)
    ref = torch.from_numpy(rnd.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = orc.bf16_to_f64(rnd)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def check_golden_store(orc):
    g = _golden("store_hand_worked.json")
    hx = lambda a: np.vectorize(lambda s: int(s, 16))(np.array(a)).astype(np.uint16)  # noqa: E731
    k = hx(g["k"])[:, None, :]
    v = hx(g["v"])[:, None, :]
    before = hx(g["k_cache_before"])[:, :, None, :]
    kc, vc = orc.store_kvcache(k, v, np.array(g["slot_mapping"]), before, before)
    assert np.array_equal(kc, hx(g["k_cache_after"])[:, :, None, :])
    assert np.array_equal(vc, hx(g["v_cache_after"])[:, :, None, :])


def check_golden_decode(orc):
    g = _golden("decode_hand_worked.json")
    hkv, d = g["num_kv_heads"], g["head_dim"]
    out = orc.decode(encode(np.array(g["q"], dtype=float)), _cache(g["k_cache"], hkv, d),
                     _cache(g["v_cache"], hkv, d), np.array(g["block_tables"]),
                     np.array(g["context_lens"]), _scale(g["scale"]))
    assert np.allclose(out, np.array(g["expected"]), rtol=0, atol=1e-12), out


def check_golden_prefill(orc):
    g = _golden("prefill_causal_hand_worked.json")
    hkv, d = g["num_kv_heads"], g["head_dim"]
    q = encode(np.array(g["q"], dtype=float))
    kp = encode(np.array(g["k_packed"], dtype=float))
    vp = encode(np.array(g["v_packed"], dtype=float))
    cq, ck = np.array(g["cu_seqlens_q"]), np.array(g["cu_seqlens_k"])
    s = _scale(g["scale"])
    for causal, key in [(True, "expected_causal"), (False, "expected_full")]:
        want = np.array(g[key])
        got = orc.prefill_varlen(q, kp, vp, cq, ck, s, causal=causal)
        assert np.allclose(got, want, rtol=0, atol=1e-12), (causal, got)
        got = orc.prefill_varlen(q, _cache(g["k_cache"], hkv, d), _cache(g["v_cache"], hkv, d),
                                 cq, ck, s, causal=causal, block_table=np.array(g["block_table"]))
        assert np.allclose(got, want, rtol=0, atol=1e-12), (causal, "table", got)


# --------------------------------------------------------------------------- store


def check_slot_of(orc):
    # hand-worked: block list [2, 0], block_size 2 -> positions 0,1,2 at slots 4,5,0
    assert [orc.slot_of([2, 0], p, 2) for p in range(3)] == [4, 5, 0]
    # block list [7, 3, 9], block_size 256: position 300 is row 44 of block 3
    assert orc.slot_of([7, 3, 9], 300, 256) == 3 * 256 + 44
    assert orc.slot_of([7, 3, 9], 0, 256) == 7 * 256
    assert orc.slot_of([7, 3, 9], 767, 256) == 9 * 256 + 255


def check_store_bruteforce(orc, seed=0):
    rng = np.random.default_rng(seed)
    nb, bs, hkv, d, t = 6, 5, 2, 3, 17
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[rng.random(t) < 0.2] = -1
    slots[[3, 8, 11]] = [nb * bs, nb * bs + 7, 2**31 - 1]  # no such slot: nothing stored
    k, v = _rand(rng, (t, hkv, d)), _rand(rng, (t, hkv, d))
    kc0 = rng.integers(0, 1 << 16, (nb, bs, hkv, d)).astype(np.uint16)
    vc0 = rng.integers(0, 1 << 16, (nb, bs, hkv, d)).astype(np.uint16)
    kc, vc = orc.store_kvcache(k, v, slots, kc0, vc0)
    want_k, want_v = kc0.reshape(nb * bs, hkv, d).copy(), vc0.reshape(nb * bs, hkv, d).copy()
    ok = (slots >= 0) & (slots < nb * bs)
    want_k[slots[ok]] = k[ok]
    want_v[slots[ok]] = v[ok]
    assert np.array_equal(kc.reshape(nb * bs, hkv, d), want_k)
    assert np.array_equal(vc.reshape(nb * bs, hkv, d), want_v)
    # the inputs are left untouched
    assert not np.shares_memory(kc, kc0)


# --------------------------------------------------------------------------- paging


def check_contiguous_equals_paged(orc, seed=1):
    rng = np.random.default_rng(seed)
    lengths, hq, hkv, d, bs = [1, 7, 12, 3], 4, 2, 8, 4
    kc, vc, tables, pk, pv = _paged_case(rng, lengths, hkv, d, bs)
    q = _rand(rng, (len(lengths), hq, d))
    scale = 0.3
    paged = orc.decode(q, kc, vc, tables, np.array(lengths), scale)
    # the same sequences laid out contiguously, blocks in order, no NaN filler
    need = [-(-n // bs) for n in lengths]
    kc2, vc2, tables2, _, _ = _paged_case(np.random.default_rng(99), lengths, hkv, d, bs,
                                          perm=np.arange(sum(need) + 2), fill_nan=False)
    for i, n in enumerate(lengths):
        for p in range(n):
            kc2[tables2[i, p // bs], p % bs] = pk[i][p]
            vc2[tables2[i, p // bs], p % bs] = pv[i][p]
    contiguous = orc.decode(q, kc2, vc2, tables2, np.array(lengths), scale)
    assert np.array_equal(paged, contiguous)
    # prefill through the table equals prefill over packed rows
    cu = np.concatenate([[0], np.cumsum(lengths)])
    qp = _rand(rng, (int(cu[-1]), hq, d))
    packed = orc.prefill_varlen(qp, np.concatenate(pk), np.concatenate(pv), cu, cu, scale)
    table = orc.prefill_varlen(qp, kc, vc, cu, cu, scale, block_table=tables)
    assert np.array_equal(packed, table)


def check_permutation_invariance(orc, block_size=3, seed=2):
    rng = np.random.default_rng(seed)
    lengths, hq, hkv, d = [5, 1, 9], 2, 1, 4
    kc, vc, tables, _, _ = _paged_case(rng, lengths, hkv, d, block_size)
    q = _rand(rng, (len(lengths), hq, d))
    base = orc.decode(q, kc, vc, tables, np.array(lengths), 0.7)
    nb = kc.shape[0]
    sigma = rng.permutation(nb)               # block b moves to sigma[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[sigma], vc2[sigma] = kc, vc
    tables2 = np.where(tables >= 0, sigma[np.maximum(tables, 0)], -1)
    moved = orc.decode(q, kc2, vc2, tables2, np.array(lengths), 0.7)
    assert np.array_equal(base, moved)


# --------------------------------------------------------------------------- softmax facts


def check_identical_keys_mean(orc, seed=3):
    rng = np.random.default_rng(seed)
    n, d = 11, 8
    key = _rand(rng, (1, 1, d))
    kc = np.repeat(key[None], n, axis=1).reshape(1, n, 1, d)
    vc = _rand(rng, (1, n, 1, d))
    q = _rand(rng, (1, 1, d))
    out = orc.decode(q, kc, vc, np.array([[0]]), np.array([n]), 1.3)
    assert np.allclose(out[0, 0], _f64(vc[0, :, 0]).mean(axis=0), rtol=0, atol=1e-12)


def check_one_token(orc, seed=4):
    rng = np.random.default_rng(seed)
    d = 16
    kc, vc = _rand(rng, (3, 2, 1, d)), _rand(rng, (3, 2, 1, d))
    q = _rand(rng, (1, 2, d))
    out = orc.decode(q, kc, vc, np.array([[2]]), np.array([1]), 0.25)
    assert np.array_equal(out[0, 0], _f64(vc[2, 0, 0])) and np.array_equal(out[0, 1], _f64(vc[2, 0, 0]))


def check_two_token_closed_form(orc, seed=5):
    rng = np.random.default_rng(seed)
    d, scale = 6, 0.37
    kc, vc = _rand(rng, (1, 2, 1, d)), _rand(rng, (1, 2, 1, d))
    q = _rand(rng, (1, 1, d))
    qf, k1, k2 = _f64(q[0, 0]), _f64(kc[0, 0, 0]), _f64(kc[0, 1, 0])
    v1, v2 = _f64(vc[0, 0, 0]), _f64(vc[0, 1, 0])
    s1 = scale * sum(float(a) * float(b) for a, b in zip(qf, k1))
    s2 = scale * sum(float(a) * float(b) for a, b in zip(qf, k2))
    e1, e2 = math.exp(s1), math.exp(s2)
    want = [(e1 * a + e2 * b) / (e1 + e2) for a, b in zip(v1, v2)]
    out = orc.decode(q, kc, vc, np.array([[0]]), np.array([2]), scale)
    assert np.allclose(out[0, 0], want, rtol=0, atol=1e-12)


def check_key_shift_and_zero_scale(orc, seed=6):
    rng = np.random.default_rng(seed)
    n, d = 9, 8
    # small integers keep K + c exact in bf16
    kint = rng.integers(-4, 5, (1, n, 1, d)).astype(float)
    c = rng.integers(-4, 5, d).astype(float)
    vc = _rand(rng, (1, n, 1, d))
    q = encode(rng.integers(-3, 4, (1, 1, d)).astype(float))
    table, lens = np.array([[0]]), np.array([n])
    a = orc.decode(q, encode(kint), vc, table, lens, 0.21)
    b = orc.decode(q, encode(kint + c), vc, table, lens, 0.21)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    z = orc.decode(q, encode(kint), vc, table, lens, 0.0)
    assert np.allclose(z[0, 0], _f64(vc[0, :, 0]).mean(axis=0), rtol=0, atol=1e-12)


def check_negative_scale_is_negated_query(orc, seed=13):
    # softmax(-s q.k) = softmax(s (-q).k): negating a bf16 query flips its sign bits, and the fp64 scores of
    # the two forms are equal bit for bit, so decode and prefill give identical outputs
    rng = np.random.default_rng(seed)
    kc, vc, table, _, _ = _paged_case(rng, [5, 17], 2, 8, 4)
    lens = np.array([5, 17])
    q = _rand(rng, (2, 4, 8))
    neg = q ^ np.uint16(0x8000)
    assert np.array_equal(orc.decode(q, kc, vc, table, lens, -0.3), orc.decode(neg, kc, vc, table, lens, 0.3))
    n = 6
    qp, kp, vp = _rand(rng, (n, 4, 8)), _rand(rng, (n, 2, 8)), _rand(rng, (n, 2, 8))
    cu = np.array([0, 2, n])
    a = orc.prefill_varlen(qp, kp, vp, cu, cu, -0.3)
    b = orc.prefill_varlen(qp ^ np.uint16(0x8000), kp, vp, cu, cu, 0.3)
    assert np.array_equal(a, b)


def check_zero_context(orc, seed=7):
    rng = np.random.default_rng(seed)
    kc, vc = _rand(rng, (2, 4, 1, 4)), _rand(rng, (2, 4, 1, 4))
    q = _rand(rng, (2, 2, 4))
    out = orc.decode(q, kc, vc, np.array([[1], [-1]]), np.array([3, 0]), 0.5)
    assert np.array_equal(out[1], np.zeros((2, 4)))
    assert np.all(np.isfinite(out[0]))


# --------------------------------------------------------------------------- GQA


def check_gqa_mapping(orc):
    # kv head g holds constant V = g + 1; query head h must read kv head h // G
    for hq, hkv in [(4, 2), (6, 3), (8, 2)]:
        d, n = 4, 5
        kc = encode(np.zeros((1, n, hkv, d)))
        vc = encode(np.broadcast_to(np.arange(1, hkv + 1, dtype=float)[None, None, :, None], (1, n, hkv, d)))
        q = encode(np.ones((1, hq, d)))
        out = orc.decode(q, kc, vc, np.array([[0]]), np.array([n]), 0.5)
        group = hq // hkv
        want = np.array([[h // group + 1.0] * d for h in range(hq)])
        assert np.array_equal(out[0], want), (hq, hkv, out[0])


def check_g1_is_mha(orc, seed=8):
    rng = np.random.default_rng(seed)
    lengths, hq, hkv, d, bs = [6, 2], 6, 2, 4, 4
    kc, vc, tables, _, _ = _paged_case(rng, lengths, hkv, d, bs)
    q = _rand(rng, (2, hq, d))
    grouped = orc.decode(q, kc, vc, tables, np.array(lengths), 0.4)
    group = hq // hkv
    idx = [h // group for h in range(hq)]
    mha = orc.decode(q, kc[:, :, idx], vc[:, :, idx], tables, np.array(lengths), 0.4)
    assert np.array_equal(grouped, mha)


# --------------------------------------------------------------------------- causal / prefix


def check_prefill_last_row_is_decode(orc, seed=9):
    rng = np.random.default_rng(seed)
    lengths, hq, hkv, d, bs = [4, 9, 1], 4, 2, 8, 4
    kc, vc, tables, pk, pv = _paged_case(rng, lengths, hkv, d, bs)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    qp = _rand(rng, (int(cu[-1]), hq, d))
    pre = orc.prefill_varlen(qp, np.concatenate(pk), np.concatenate(pv), cu, cu, 0.3)
    last = qp[cu[1:] - 1]
    dec = orc.decode(last, kc, vc, tables, np.array(lengths), 0.3)
    assert np.allclose(pre[cu[1:] - 1], dec, rtol=0, atol=1e-12)


def check_prefix_rows_equal_full(orc, seed=10):
    rng = np.random.default_rng(seed)
    prefix, news, hq, hkv, d, bs = 7, [3, 5], 2, 1, 4, 4
    totals = [prefix + m for m in news]
    kc, vc, tables, pk, pv = _paged_case(rng, totals, hkv, d, bs)
    qs = [_rand(rng, (n, hq, d)) for n in totals]
    scale = 0.45
    cu_full = np.concatenate([[0], np.cumsum(totals)])
    full = orc.prefill_varlen(np.concatenate(qs), np.concatenate(pk), np.concatenate(pv),
                              cu_full, cu_full, scale)
    cu_q = np.concatenate([[0], np.cumsum(news)])
    q_new = np.concatenate([qs[i][prefix:] for i in range(len(news))])
    cached = orc.prefill_varlen(q_new, kc, vc, cu_q, cu_full, scale, block_table=tables)
    want = np.concatenate([full[cu_full[i] + prefix:cu_full[i + 1]] for i in range(len(news))])
    assert np.allclose(cached, want, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- independent implementations


def _sdpa(q, k, v, last_key, scale):
    """torch SDPA in fp64; q [m, H, D], k/v [n, H, D] (kv heads already expanded)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    mask = torch.from_numpy(np.arange(k.shape[0])[None, :] <= np.asarray(last_key)[:, None])
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def check_against_sdpa(orc, seed=11):
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 6, 2, 8, 4
    group = hq // hkv
    expand = [h // group for h in range(hq)]
    scale = 1.0 / math.sqrt(d)
    # decode
    lengths = [1, 5, 13, 8]
    kc, vc, tables, pk, pv = _paged_case(rng, lengths, hkv, d, bs)
    q = _rand(rng, (len(lengths), hq, d))
    out = orc.decode(q, kc, vc, tables, np.array(lengths), scale)
    for b, n in enumerate(lengths):
        want = _sdpa(_f64(q[b])[None], _f64(pk[b])[:, expand], _f64(pv[b])[:, expand], [n - 1], scale)
        assert np.allclose(out[b], want[0], rtol=0, atol=1e-12)
    # prefill with fewer queries than keys, packed and through the table
    nq = [1, 3, 13, 2]
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    cu_k = np.concatenate([[0], np.cumsum(lengths)])
    qp = _rand(rng, (int(cu_q[-1]), hq, d))
    for causal in (True, False):
        a = orc.prefill_varlen(qp, np.concatenate(pk), np.concatenate(pv), cu_q, cu_k, scale, causal)
        t = orc.prefill_varlen(qp, kc, vc, cu_q, cu_k, scale, causal, block_table=tables)
        for i in range(len(nq)):
            n, m = lengths[i], nq[i]
            last = [n - m + j if causal else n - 1 for j in range(m)]
            want = _sdpa(_f64(qp[cu_q[i]:cu_q[i + 1]]), _f64(pk[i])[:, expand], _f64(pv[i])[:, expand],
                         last, scale)
            assert np.allclose(a[cu_q[i]:cu_q[i + 1]], want, rtol=0, atol=1e-12)
            assert np.allclose(t[cu_q[i]:cu_q[i + 1]], want, rtol=0, atol=1e-12)


def check_against_bruteforce(orc, seed=12):
    """Pure-Python loops over tokens, heads and dims (math.exp), tiny sizes."""
    rng = np.random.default_rng(seed)
    hq, hkv, d, bs = 2, 1, 3, 2
    lengths = [3, 4]
    kc, vc, tables, pk, pv = _paged_case(rng, lengths, hkv, d, bs)
    q = _rand(rng, (2, hq, d))
    scale = 0.9
    out = orc.decode(q, kc, vc, tables, np.array(lengths), scale)
    for b, n in enumerate(lengths):
        for h in range(hq):
            qv = [float(x) for x in _f64(q[b, h])]
            scores = []
            for t in range(n):
                blk, row = int(tables[b][t // bs]), t % bs
                kv = [float(x) for x in _f64(kc[blk, row, h // (hq // hkv)])]
                scores.append(scale * sum(qv[i] * kv[i] for i in range(d)))
            top = max(scores)
            w = [math.exp(s - top) for s in scores]
            for i in range(d):
                num = 0.0
                for t in range(n):
                    blk, row = int(tables[b][t // bs]), t % bs
                    num += w[t] * float(_f64(vc[blk, row, h // (hq // hkv)])[i])
                assert abs(out[b, h, i] - num / sum(w)) <= 1e-12


ALL_CHECKS = [
    check_bf16_widen, check_golden_store, check_golden_decode, check_golden_prefill,
    check_slot_of, check_store_bruteforce, check_contiguous_equals_paged, check_permutation_invariance,
    check_identical_keys_mean, check_one_token, check_two_token_closed_form,
    check_key_shift_and_zero_scale, check_negative_scale_is_negated_query, check_zero_context, check_gqa_mapping, check_g1_is_mha,
    check_prefill_last_row_is_decode, check_prefix_rows_equal_full, check_against_sdpa,
    check_against_bruteforce,
]
