"""The QK-norm + rotary oracle against its pins, and planted mistakes against the pins (CPU only)."""

import os
import types

import pytest

import oracle.norm_rope as orc
from tests import oracle_pins_rope as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "norm_rope.py")

MUTANTS = {
    "rotation_sign": ("a * cos - b * sin", "a * cos + b * sin"),
    "interleaved_pairs": ("a, b = x[..., :h], x[..., h:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    "sum_not_mean": ("ms = np.mean(x * x, axis=-1, keepdims=True)", "ms = np.sum(x * x, axis=-1, keepdims=True)"),
    "eps_outside_sqrt": ("np.sqrt(ms + eps)", "(np.sqrt(ms) + eps)"),
    "rotate_before_norm": (
        "return rotate_half_pairs(qn, cos, sin), rotate_half_pairs(kn, cos, sin), v",
        "return (rms_norm(rotate_half_pairs(q, cos, sin), bf16_to_f64(q_weight), eps),\n"
        "            rms_norm(rotate_half_pairs(k, cos, sin), bf16_to_f64(k_weight), eps), v)"),
    "k_takes_q_weight": ("kn = rms_norm(k, bf16_to_f64(k_weight), eps)", "kn = rms_norm(k, bf16_to_f64(q_weight), eps)"),
    "k_from_v_heads": ("k = bf16_to_f64(heads[:, num_q_heads:num_q_heads + num_kv_heads])",
                       "k = bf16_to_f64(heads[:, num_q_heads + num_kv_heads:])"),
    "v_from_k_heads": ("v = heads[:, num_q_heads + num_kv_heads:].copy()",
                       "v = heads[:, num_q_heads:num_q_heads + num_kv_heads].copy()"),
    "cos_sin_swapped": ("cos = table[:, None, :h]\n    sin = table[:, None, h:]",
                        "cos = table[:, None, h:]\n    sin = table[:, None, :h]"),
    "position_off_by_one": ("[np.asarray(positions, dtype=np.int64)]", "[np.asarray(positions, dtype=np.int64) - 1]"),
}


def _mutant(old, new):
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    src = src.replace("from .paged_attention import", "from oracle.paged_attention import")
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_rope_mutant")
    exec(compile(src.replace(old, new), "oracle_rope_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(orc)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # an assertion, or a crash on a bad index
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
