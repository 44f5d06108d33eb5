"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Each mutant is the oracle's source with one plausible slip written in (a wrong
index, sign, operand or alignment). A pin set that lets any of them through
would not be pinning the oracle.
"""

import os
import types

import pytest

from tests import oracle_pins as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "paged_attention.py")

MUTANTS = {
    "gqa_modulo_mapping": ("g = h // group", "g = h % hkv"),
    "causal_top_left": ("last_key = [nk - nq + j for j in range(nq)]", "last_key = [j for j in range(nq)]"),
    "dropped_scale": ("scores = scale * (q @ keys.T)", "scores = (q @ keys.T)"),
    "exp_sign": ("w = np.exp(s - s.max())", "w = np.exp(s.max() - s)"),
    "gather_row_off_by_one": ("p % block_size] for p in range(n)", "(p + 1) % block_size] for p in range(n)"),
    "keys_as_values": ("out[j] = (w @ values[allowed[j]]) / w.sum()", "out[j] = (w @ keys[allowed[j]]) / w.sum()"),
    "decode_excludes_new_token": ("[length - 1])[0]", "[length - 2])[0]"),
    "mask_strict": ("allowed = np.arange(n)[None, :] <= np.asarray(last_key)[:, None]",
                    "allowed = np.arange(n)[None, :] < np.asarray(last_key)[:, None]"),
    "widen_shift": ("<< np.uint32(16)", "<< np.uint32(15)"),
    "normalise_by_max": ("/ w.sum()", "/ w.max()"),
    "store_transposed_index": ("kc[s // block_size, s % block_size] = k[t]",
                               "kc[s % block_size, s // block_size] = k[t]"),
    "store_skips_slot_zero": ("if s < 0 or s >= capacity:", "if s <= 0 or s >= capacity:"),
    "store_capacity_off_by_one": ("if s < 0 or s >= capacity:", "if s < 0 or s > capacity:"),
    "wrong_query_head": ("qb[h][None, :]", "qb[g][None, :]"),
    "gather_block_index": ("cache[int(block_list[p // block_size]), p % block_size]",
                           "cache[int(block_list[p % block_size]) if p % block_size < len(block_list) else 0, p % block_size]"),
    "slot_row_from_division": ("* block_size + pos % block_size", "* block_size + pos // block_size"),
    "packed_keys_offset": ("keys = bf16_to_f64(k[k0:k1])", "keys = bf16_to_f64(k[q0:q0 + nk])"),
}


def _mutant(old, new):
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


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
