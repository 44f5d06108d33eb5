"""The block-manager model against its pins, and planted mistakes against the pins (CPU only)."""

import os
import types

import pytest

import oracle.block_manager as orc
from tests import oracle_pins_blocks as pins

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "block_manager.py")

MUTANTS = {
    "hash_ignores_prefix": ("block_hash(blk, h)", "block_hash(blk, 0)"),
    "free_to_front": ("self.free.append(b)", "self.free.insert(0, b)"),
    "free_in_table_order": ("for b in reversed(s[\"table\"]):", "for b in s[\"table\"]:"),
    "whole_prompt_cacheable": ("range((n - 1) // bs if n > 0 else 0)", "range(n // bs)"),
    "hit_not_counted": ("            self.ref[b] += 1\n", "            pass\n"),
    "append_block_boundary": ("        if s[\"len\"] % bs == 0:\n            if not self.free:",
                              "        if s[\"len\"] % bs == 1:\n            if not self.free:"),
    "filled_block_not_hashed": ("        if s[\"len\"] % bs == 0:\n            b = s[\"table\"][-1]",
                                "        if False:\n            b = s[\"table\"][-1]"),
    "capacity_ignores_free_hits": ("nblocks - len(hits) + from_free > len(self.free)",
                                   "nblocks - len(hits) > len(self.free)"),
    "take_from_back": ("b = self.free.pop(0)", "b = self.free.pop()"),
}


def _mutant(old, new):
    with open(SRC_PATH, encoding="utf-8") as f:
        src = f.read()
    assert old in src, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_blocks_mutant")
    exec(compile(src.replace(old, new), "oracle_blocks_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(orc)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_invariants_more_seeds(seed):
    pins.check_invariants_random(orc, seed=seed)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception:  # an assertion, or a crash
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
