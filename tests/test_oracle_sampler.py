"""The sampler oracle against its pins, and planted mistakes against the pins (CPU only)."""

import os
import types

import pytest

import oracle.sampler as orc
from tests import oracle_pins_sampler as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sampler.py")

MUTANTS = {
    "philox_nine_rounds": ("for _ in range(10):", "for _ in range(9):"),
    "philox_lo_hi_swapped": ("x = [(p1 >> _S32) ^ x[1] ^ k0, p1 & _LO32, (p0 >> _S32) ^ x[3] ^ k1, p0 & _LO32]",
                             "x = [(p1 & _LO32) ^ x[1] ^ k0, p1 >> _S32, (p0 & _LO32) ^ x[3] ^ k1, p0 >> _S32]"),
    "philox_multipliers_swapped": ("p0 = M0 * x[0]", "p0 = M1 * x[0]"),
    "key_not_bumped": ("        k1 = (k1 + W1) & _LO32\n", "        k1 = k1\n"),
    "seed_high_half_dropped": ("key[..., 1] = np.uint64(sd >> 32)", "key[..., 1] = np.uint64(0)"),
    "offset_high_half_dropped": ("np.full_like(j, np.uint64(off >> 32))", "np.zeros_like(j)"),
    "uniform_low_bits": ("fields[..., 3 * h] = x >> np.uint64(43)", "fields[..., 3 * h] = x & mask"),
    "fields_swapped": ("fields[..., 3 * h] = x >> np.uint64(43)\n        fields[..., 3 * h + 1] = (x >> np.uint64(22))",
                       "fields[..., 3 * h + 1] = x >> np.uint64(43)\n        fields[..., 3 * h] = (x >> np.uint64(22))"),
    "third_field_unshifted": ("fields[..., 3 * h + 2] = (x >> np.uint64(1)) & mask", "fields[..., 3 * h + 2] = x & mask"),
    "words_paired_wrongly": ("halves = [(w[..., 1] << _S32) | w[..., 0], (w[..., 3] << _S32) | w[..., 2]]",
                             "halves = [(w[..., 0] << _S32) | w[..., 1], (w[..., 3] << _S32) | w[..., 2]]"),
    "two_to_the_23": ("/ 2.0 ** 21", "/ 2.0 ** 23"),
    "counter_row_and_block_swapped": ("ctr = np.stack([j, b,", "ctr = np.stack([b, j,"),
    "noise_is_uniform": ("e = -np.log(u)", "e = u"),
    "multiplies_by_noise": ("- np.log(e)", "+ np.log(e)"),
    "temperature_multiplies": ("lg / t[:, None]", "lg * t[:, None]"),
}


def _mutant(old, new):
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_sampler_mutant")
    exec(compile(src.replace(old, new), "oracle_sampler_mutant", "exec"), mod.__dict__)
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
        except Exception:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
