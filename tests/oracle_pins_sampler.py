"""Checks that pin the Gumbel-max sampler oracle to facts other than itself.

Each ``check_*`` takes a module exposing ``philox4x32``, ``uniforms``,
``scores`` and ``sample`` (the real ``oracle.sampler`` or a mutant). The
facts: rocRAND's Philox4x32-10 engine (its header, compiled here for the host:
an independent implementation of the same generator), the stated
word-to-uniform map applied to rocRAND's words, the literal definition
argmax softmax(l/T)/E with scipy's softmax, token frequencies that must follow
softmax(l/T) (chi-square), and the limits of a dominant logit and of a small
temperature.
"""

from __future__ import annotations

import functools
import os
import shutil
import subprocess
import tempfile

import numpy as np
import scipy.special
import scipy.stats

_HERE = os.path.dirname(os.path.abspath(__file__))


@functools.lru_cache(maxsize=1)
def _reference_binary() -> str:
    """Build tests/philox_ref.cpp (rocRAND's header engine, host code) once per session."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    out = os.path.join(tempfile.mkdtemp(prefix="philox_ref_"), "philox_ref")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", os.path.join(_HERE, "philox_ref.cpp"),
                    "-o", out], check=True, capture_output=True, timeout=300)
    return out


def reference_blocks(triples):
    """rocRAND's Philox4x32-10 block for each (seed, subsequence, c): counter (c lo, c hi, sub lo, sub hi),
    key (seed lo, seed hi). Returns uint64 [n, 4] holding 32-bit words."""
    text = "".join(f"{int(s)} {int(u)} {int(c)}\n" for s, u, c in triples)
    res = subprocess.run([_reference_binary()], input=text, capture_output=True, text=True, check=True, timeout=60)
    return np.array([[int(w) for w in line.split()] for line in res.stdout.splitlines()], dtype=np.uint64)


def check_philox_matches_rocrand(orc, seed=0):
    rng = np.random.default_rng(seed)
    triples = [(int(rng.integers(0, 2 ** 63)) * 2 + int(rng.integers(0, 2)), int(rng.integers(0, 2 ** 63)),
                int(rng.integers(0, 2 ** 62))) for _ in range(24)]
    # (the engine skips 4 c numbers in a 64-bit count, so c stays below 2^62)
    triples += [(0, 0, 0), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 62 - 1), (1, 2 ** 32 + 5, 2 ** 32 - 1)]
    want = reference_blocks(triples)
    for (sd, sub, c), w in zip(triples, want):
        ctr = np.array([[c % 2 ** 32, c >> 32, sub % 2 ** 32, sub >> 32]], dtype=np.uint64)
        key = np.array([[sd % 2 ** 32, sd >> 32]], dtype=np.uint64)
        assert np.array_equal(orc.philox4x32(ctr, key)[0], w), (sd, sub, c)


def check_uniforms_from_reference_words(orc):
    # element i of row b: field i % 6 of the block at counter (i // 6, b, offset lo, offset hi), key
    # (seed lo, seed hi); fields 0..2 are bits 63..43, 42..22, 21..1 of w1 * 2^32 + w0, fields 3..5 the
    # same bits of w3 * 2^32 + w2; u = (field + 1/2) / 2^21
    seed, offset, rows, vocab = 0x0123456789ABCDEF, 2 ** 40 + 7, 3, 61
    u = orc.uniforms(rows, vocab, seed, offset)
    assert u.shape == (rows, vocab)
    nblk = -(-vocab // 6)
    for b in range(rows):
        # the engine's counter (c lo, c hi, sub lo, sub hi) = (j, b, offset lo, offset hi): c = j + 2^32 b
        words = reference_blocks([(seed, offset, j + (b << 32)) for j in range(nblk)])
        for i in range(vocab):
            w = words[i // 6]
            x = int(w[1]) << 32 | int(w[0]) if (i % 6) < 3 else int(w[3]) << 32 | int(w[2])
            field = (x >> (43 - 21 * (i % 3))) % (1 << 21)
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


ALL_CHECKS = [check_philox_matches_rocrand, check_uniforms_from_reference_words, check_literal_definition,
              check_frequencies_follow_softmax, check_dominant_logit_and_small_temperature,
              check_reproducible_and_distinct_streams]
