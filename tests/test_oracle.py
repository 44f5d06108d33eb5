"""The oracle against its pins (CPU only)."""

import pytest
from hypothesis import given, settings, strategies as st

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)


@settings(max_examples=25, deadline=None)
@given(block_size=st.sampled_from([1, 2, 3, 4, 5, 256]), seed=st.integers(0, 10_000))
def test_permutation_invariance_any_block_size(block_size, seed):
    pins.check_permutation_invariance(oracle, block_size=block_size, seed=seed)


@settings(max_examples=10, deadline=None)
@given(seed=st.integers(0, 10_000))
def test_sdpa_random_seeds(seed):
    pins.check_against_sdpa(oracle, seed=seed)


@settings(max_examples=10, deadline=None)
@given(seed=st.integers(0, 10_000))
def test_store_random_seeds(seed):
    pins.check_store_bruteforce(oracle, seed=seed)
