"""The attention pass rule itself (CPU): literal bounds, and the one place a bf16 output cannot meet
the absolute bound."""

import numpy as np
import pytest
import torch

from tests import parity


@pytest.fixture(autouse=True)
def _keep_record_clean():
    # these cases exercise the rule, they are not parity results: keep them out of the run's summary
    saved = dict(parity.RECORD)
    yield
    parity.RECORD.clear()
    parity.RECORD.update(saved)


def test_bf16_neighbours_bracket_torch_rounding():
    x = np.random.default_rng(0).standard_normal(200_000) * 6
    lo, hi = parity.bf16_neighbours(x)
    rounded = torch.tensor(x).to(torch.bfloat16).double().numpy()
    assert np.all((rounded == lo) | (rounded == hi))
    assert np.all(np.abs(lo) <= np.abs(x)) and np.all(np.abs(x) < np.abs(hi))


def test_unattainable_only_at_or_above_four():
    # below 4 the nearest bf16 value is at most 2^-7 away, so 1e-2 is always reachable
    x = np.linspace(-3.999, 3.999, 400_001)
    stats = parity.attention_errors(x, x)
    assert stats["n_bf16_unattainable"] == 0
    y = np.array([4.326])  # neighbours 4.3125 and 4.34375, both more than 1e-2 away
    assert parity.attention_errors(y, y)["n_bf16_unattainable"] == 1


def _bf(vals):
    return torch.tensor(vals, dtype=torch.bfloat16)


def test_literal_bounds_pass_and_fail():
    parity.assert_attention_close(_bf([1.0, 0.0]), np.array([1.0049, 0.0099]), "ok")
    with pytest.raises(AssertionError, match="max abs"):
        parity.assert_attention_close(_bf([0.0]), np.array([0.0101]), "abs")
    with pytest.raises(AssertionError, match="max abs"):
        # 2e-2 relative would admit it; the absolute bound does not
        parity.assert_attention_close(_bf([3.0]), np.array([3.0118]), "abs above 0.5")


def test_unattainable_element_must_be_a_bf16_neighbour():
    parity.assert_attention_close(_bf([4.3125]), np.array([4.326]), "lower neighbour")
    parity.assert_attention_close(_bf([4.34375]), np.array([4.326]), "upper neighbour")
    with pytest.raises(AssertionError, match="neighbour"):
        parity.assert_attention_close(_bf([4.28125]), np.array([4.326]), "two steps away")


def test_non_finite_output_fails():
    with pytest.raises(AssertionError, match="non-finite"):
        parity.assert_attention_close(_bf([float("nan")]), np.array([0.0]), "nan")
