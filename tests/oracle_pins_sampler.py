"""Checks that pin the Gumbel-max sampler oracle to facts other than itself.

Each ``check_*`` takes a module exposing ``philox4x64``, ``uniforms``,
``scores`` and ``sample`` (the real ``oracle.sampler`` or a mutant). The
facts: numpy's own Philox4x64-10 generator, the stated word-to-uniform map
applied to numpy's words, the literal definition argmax softmax(l/T)/E with
scipy's softmax, token frequencies that must follow softmax(l/T) (chi-square),
and the limits of a dominant logit and of a small temperature.
"""

from __future__ import annotations

import numpy as np
import scipy.special
import scipy.stats


def _numpy_block(counter, key):
    """numpy's Philox4x64-10 block at `counter` (numpy steps the counter before each block)."""
    c = [int(x) for x in counter]
    c[0] -= 1
    return np.random.Philox(counter=c, key=[int(k) for k in key]).random_raw(4)


def check_philox_matches_numpy(orc, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        ctr = rng.integers(1, 2 ** 63, 4, dtype=np.uint64)
        key = rng.integers(0, 2 ** 63, 2, dtype=np.uint64)
        got = orc.philox4x64(ctr[None, :], key[None, :])[0]
        assert np.array_equal(got, _numpy_block(ctr, key))


def check_uniforms_from_numpy_words(orc):
    # element i of row b: 21-bit field of word (i // 3) % 4 of the block at counter
    # (i // 12, b, offset, 0), key (seed, 0): bits 63..43, 42..22 or 21..1 for i % 3 = 0, 1, 2;
    # u = (field + 1/2) / 2^21. Blocks j >= 1 are compared (numpy cannot start below counter 0).
    seed, offset, rows, vocab = 123456789, 7, 3, 61
    u = orc.uniforms(rows, vocab, seed, offset)
    assert u.shape == (rows, vocab)
    for b in range(rows):
        for i in range(12, vocab):
            w = int(_numpy_block([i // 12, b, offset, 0], [seed, 0])[(i // 3) % 4])
            field = (w >> (43 - 21 * (i % 3))) % (1 << 21)
            assert u[b, i] == (field + 0.5) / 2.0 ** 21, (b, i)
    assert np.all(u > 0) and np.all(u < 1)
    assert np.array_equal(u.astype(np.float32).astype(np.float64), u)  # exact in fp32


def check_literal_definition(orc, seed=1):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((6, 37)) * 3
    t = np.array([0.3, 0.7, 1.0, 1.5, 2.0, 1e-3])
    u = orc.uniforms(6, 37, 99, 4)
    p = scipy.special.softmax(lg / t[:, None], axis=1)
    want = np.argmax(p / (-np.log(u)), axis=1)
    assert np.array_equal(orc.sample(lg, t, 99, 4), want)


def check_frequencies_follow_softmax(orc):
    lg = np.array([1.0, 0.0, -0.5, 2.0, 0.3])
    rows = 20000
    for t in (0.5, 1.0, 2.0):
        toks = orc.sample(np.tile(lg, (rows, 1)), np.full(rows, t), 2024, 0)
        counts = np.bincount(toks, minlength=len(lg))
        expected = scipy.special.softmax(lg / t) * rows
        assert scipy.stats.chisquare(counts, expected).pvalue > 1e-3, (t, counts, expected)


def check_dominant_logit_and_small_temperature(orc, seed=2):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((50, 100))
    lg[np.arange(50), rng.integers(0, 100, 50)] += 60.0  # probability ~ 1 - 1e-24
    assert np.array_equal(orc.sample(lg, np.ones(50), 5, 0), np.argmax(lg, axis=1))
    lg2 = rng.standard_normal((50, 1000))
    assert np.array_equal(orc.sample(lg2, np.full(50, 1e-7), 6, 1), np.argmax(lg2, axis=1))


def check_reproducible_and_distinct_streams(orc):
    a = orc.uniforms(4, 64, 1, 0)
    assert np.array_equal(a, orc.uniforms(4, 64, 1, 0))
    assert not np.array_equal(a, orc.uniforms(4, 64, 2, 0))   # another seed
    assert not np.array_equal(a, orc.uniforms(4, 64, 1, 1))   # another offset (step)
    assert not np.array_equal(a[0], a[1])                      # another row


ALL_CHECKS = [check_philox_matches_numpy, check_uniforms_from_numpy_words, check_literal_definition,
              check_frequencies_follow_softmax, check_dominant_logit_and_small_temperature,
              check_reproducible_and_distinct_streams]
