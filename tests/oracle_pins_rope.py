"""Checks that pin the fp64 QK-norm + rotary oracle to facts other than itself.

Each ``check_*`` takes a module exposing ``qk_norm_rope``, ``rms_norm`` and
``rotate_half_pairs`` (the real ``oracle.norm_rope`` or a mutant) and raises
``AssertionError`` when the module breaks the fact. The facts: a hand-worked
golden example (``tests/golden/qk_norm_rope_hand_worked.json``), exact
invariants of a normalisation followed by a rotation, torch's own
``rms_norm``, the relative-position property that defines rotary embeddings,
and the routing of heads, weights and V.
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch

from workloads.bf16 import decode_f32, encode
from workloads.rope import cos_sin_table

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(bits):
    return decode_f32(bits).astype(np.float64)


def _qkv(rng, t, hq, hkv, d):
    return encode(rng.standard_normal((t, (hq + 2 * hkv) * d)))


def check_golden(orc):
    with open(os.path.join(GOLDEN, "qk_norm_rope_hand_worked.json"), encoding="utf-8") as f:
        g = json.load(f)
    q, k, v = orc.qk_norm_rope(encode(g["qkv"]), g["positions"], np.asarray(g["cos_sin"], np.float32),
                               encode(g["q_weight"]), encode(g["k_weight"]), g["eps"], g["num_q_heads"],
                               g["num_kv_heads"])
    np.testing.assert_allclose(q[:, 0], np.asarray(g["expected_q"]), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(k[:, 0], np.asarray(g["expected_k"]), rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(_f64(v[:, 0]), np.asarray(g["expected_v"]))


def check_unit_rms(orc, seed=0):
    # weight 1, eps 0: every output head has mean square exactly 1 (the
    # rotation keeps each pair's length), whatever the position
    rng = np.random.default_rng(seed)
    t, hq, hkv, d = 5, 4, 2, 16
    table = cos_sin_table(64, d, base=100.0)
    ones = encode(np.ones(d))
    q, k, _ = orc.qk_norm_rope(_qkv(rng, t, hq, hkv, d), rng.integers(0, 64, t), table, ones, ones, 0.0, hq, hkv)
    np.testing.assert_allclose(np.mean(q * q, axis=-1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(np.mean(k * k, axis=-1), 1.0, rtol=1e-6)


def check_identity_row_is_torch_rms_norm(orc, seed=1):
    # a row with cos 1, sin 0 leaves only the normalisation: torch's rms_norm
    rng = np.random.default_rng(seed)
    t, hq, hkv, d, eps = 3, 2, 1, 8, 1e-3
    table = np.concatenate([np.ones((1, d // 2)), np.zeros((1, d // 2))], axis=1).astype(np.float32)
    qkv = _qkv(rng, t, hq, hkv, d)
    qw, kw = encode(1 + 0.3 * rng.standard_normal(d)), encode(1 + 0.3 * rng.standard_normal(d))
    q, k, _ = orc.qk_norm_rope(qkv, np.zeros(t, np.int64), table, qw, kw, eps, hq, hkv)
    x = torch.from_numpy(_f64(qkv).reshape(t, hq + 2 * hkv, d))
    ref_q = torch.nn.functional.rms_norm(x[:, :hq], (d,), torch.from_numpy(_f64(qw)), eps).numpy()
    ref_k = torch.nn.functional.rms_norm(x[:, hq:hq + hkv], (d,), torch.from_numpy(_f64(kw)), eps).numpy()
    np.testing.assert_allclose(q, ref_q, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(k, ref_k, rtol=1e-12, atol=1e-14)


def check_relative_position(orc, seed=2):
    # the defining property of rotary embeddings: <q at m, k at n> depends on m - n only
    rng = np.random.default_rng(seed)
    d = 32
    table = cos_sin_table(512, d, base=10000.0)
    ones = encode(np.ones(d))
    base_qkv = _qkv(rng, 1, 1, 1, d)
    qkv = np.repeat(base_qkv, 6, axis=0)
    pos = np.array([7, 3, 107, 103, 411, 407])  # three (m, n) pairs with m - n = 4
    q, k, _ = orc.qk_norm_rope(qkv, pos, table, ones, ones, 0.0, 1, 1)
    dots = [float(q[2 * i, 0] @ k[2 * i + 1, 0]) for i in range(3)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-5)
    # and the same pairs the other way round (n - m = 4) give a different value
    back = float(q[1, 0] @ k[0, 0])
    assert abs(back - dots[0]) > 1e-3


def check_rotation_composes(orc, seed=3):
    # turning by the angles of rows a and b equals turning by those of row a + b
    rng = np.random.default_rng(seed)
    d = 16
    table = cos_sin_table(64, d, base=50.0).astype(np.float64)
    x = rng.standard_normal((4, d))
    h = d // 2
    a, b = 5, 9
    once = orc.rotate_half_pairs(x, table[a + b, :h], table[a + b, h:])
    twice = orc.rotate_half_pairs(orc.rotate_half_pairs(x, table[a, :h], table[a, h:]), table[b, :h], table[b, h:])
    np.testing.assert_allclose(twice, once, rtol=1e-5, atol=1e-6)


def check_heads_weights_and_v(orc):
    # head j of q / k / v is one-hot at dimension j; with an identity row the
    # output of head j must again be one-hot at j (so each output head comes
    # from its own input head), scaled by sqrt(d) times its own weight
    d, hq, hkv = 8, 2, 2
    nh = hq + 2 * hkv
    x = np.zeros((1, nh, d))
    for j in range(nh):
        x[0, j, j] = j + 1
    table = np.concatenate([np.ones((1, d // 2)), np.zeros((1, d // 2))], axis=1).astype(np.float32)
    qw, kw = encode(np.full(d, 2.0)), encode(np.full(d, 3.0))
    q, k, v = orc.qk_norm_rope(encode(x.reshape(1, -1)), [0], table, qw, kw, 0.0, hq, hkv)
    for j in range(hq):
        expect = np.zeros(d)
        expect[j] = 2.0 * np.sqrt(d)
        np.testing.assert_allclose(q[0, j], expect, rtol=1e-12)
    for j in range(hkv):
        expect = np.zeros(d)
        expect[hq + j] = 3.0 * np.sqrt(d)
        np.testing.assert_allclose(k[0, j], expect, rtol=1e-12)
    np.testing.assert_array_equal(_f64(v[0]), x[0, hq + hkv:])


def check_eps_closed_form(orc):
    # a constant head c * 1 normalises to c / sqrt(c^2 + eps) per element
    d, c, eps = 8, 0.5, 0.75
    table = np.concatenate([np.ones((1, d // 2)), np.zeros((1, d // 2))], axis=1).astype(np.float32)
    ones = encode(np.ones(d))
    qkv = encode(np.full((1, 3 * d), c))
    q, k, _ = orc.qk_norm_rope(qkv, [0], table, ones, ones, eps, 1, 1)
    np.testing.assert_allclose(q[0, 0], c / np.sqrt(c * c + eps), rtol=1e-12)
    np.testing.assert_allclose(k[0, 0], c / np.sqrt(c * c + eps), rtol=1e-12)


def check_against_bruteforce(orc, seed=4):
    # element-by-element restatement with Python floats on a tiny input
    rng = np.random.default_rng(seed)
    t, hq, hkv, d, eps = 2, 2, 1, 4, 1e-2
    table = cos_sin_table(8, d, base=3.0)
    qkv = _qkv(rng, t, hq, hkv, d)
    qw, kw = encode(1 + rng.standard_normal(d) * 0.2), encode(1 + rng.standard_normal(d) * 0.2)
    pos = [3, 6]
    q, k, _ = orc.qk_norm_rope(qkv, pos, table, qw, kw, eps, hq, hkv)
    xs = _f64(qkv).reshape(t, hq + 2 * hkv, d)
    for ti in range(t):
        row = [float(c) for c in table[pos[ti]]]
        for hh in range(hq + hkv):
            w = _f64(qw) if hh < hq else _f64(kw)
            vec = [float(c) for c in xs[ti, hh]]
            ss = 0.0
            for c in vec:
                ss += c * c
            r = (ss / d + eps) ** 0.5
            n = [vec[i] / r * float(w[i]) for i in range(d)]
            out = [0.0] * d
            for i in range(d // 2):
                cs, sn = row[i], row[d // 2 + i]
                out[i] = n[i] * cs - n[i + d // 2] * sn
                out[i + d // 2] = n[i + d // 2] * cs + n[i] * sn
            got = q[ti, hh] if hh < hq else k[ti, hh - hq]
            np.testing.assert_allclose(got, out, rtol=1e-12, atol=1e-14)


ALL_CHECKS = [
    check_golden,
    check_unit_rms,
    check_identity_row_is_torch_rms_norm,
    check_relative_position,
    check_rotation_composes,
    check_heads_weights_and_v,
    check_eps_closed_form,
    check_against_bruteforce,
]
