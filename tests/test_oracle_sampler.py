"""The sampler oracle against its pins, and planted mistakes against the pins (CPU only)."""

import os
import types

import pytest

import oracle.sampler as orc
from tests import oracle_pins_sampler as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sampler.py")

MUTANTS = {
    "philox_nine_rounds": ("for _ in range(10):", "for _ in range(9):"),
    "philox_lo_hi_swapped": ("x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]",
                             "x = [lo1 ^ x[1] ^ k0, hi1, lo0 ^ x[3] ^ k1, hi0]"),
    "key_not_bumped": ("            k1 = k1 + W1\n", "            k1 = k1\n"),
    "uniform_low_bits": ("fields[:, 0::3] = words >> np.uint64(43)", "fields[:, 0::3] = words & mask"),
    "fields_swapped": ("fields[:, 0::3] = words >> np.uint64(43)\n    fields[:, 1::3] = (words >> np.uint64(22))",
                       "fields[:, 1::3] = words >> np.uint64(43)\n    fields[:, 0::3] = (words >> np.uint64(22))"),
    "third_field_unshifted": ("fields[:, 2::3] = (words >> np.uint64(1)) & mask", "fields[:, 2::3] = words & mask"),
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
