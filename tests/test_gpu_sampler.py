"""pa_sample_gumbel on the GPU against the fp64 oracle.

The kernel takes its argmax over fp32 scores (two hardware log2 per element),
the oracle over exact ones, so the comparison follows the rule for decisions
taken in floating point: wherever the oracle's best score leads the runner-up
by more than eps, the tokens must be equal; otherwise the kernel's token must
be an eps-argmax of the exact scores. eps = 1e-5 * (max_i |l_i / T| + 30)
(natural-log units) bounds the fp32 rounding of l / T and the relative error
of the two log2 evaluations with a wide margin.
"""

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle.sampler as osmp
import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401

pytestmark = pytest.mark.gpu


def _run(logits, temps, seed, offset, dev):
    lg = torch.as_tensor(np.ascontiguousarray(logits, dtype=np.float32)).to(dev)
    t = torch.as_tensor(np.asarray(temps, dtype=np.float32)).to(dev)
    out = pa.pa_sample_gumbel(lg, t, seed, offset)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


def _check(got, logits, temps, seed, offset):
    s = osmp.scores(logits.astype(np.float32), np.asarray(temps, dtype=np.float32), seed, offset)
    lt = np.where(np.isfinite(logits), np.abs(logits / np.maximum(np.asarray(temps, np.float64), 1e-10)[:, None]), 0)
    eps = 1e-5 * (lt.max(axis=1) + 30.0)
    best = np.argmax(s, axis=1)
    rows = np.arange(len(got))
    top = s[rows, best]
    runner = np.partition(s, -2, axis=1)[:, -2] if s.shape[1] > 1 else np.full(len(got), -np.inf)
    separated = top - runner > eps
    assert np.array_equal(got[separated], best[separated]), "token differs where the decision is clear"
    assert np.all(s[rows, got] >= top - eps), "token is not an eps-argmax of the exact scores"
    return int((~separated).sum())


@pytest.mark.parametrize("vocab", [1, 7, 8, 9, 11, 12, 13, 8191, 8192, 8193, 12287, 12288, 12289, 20000])
def test_sampler_small(dev, vocab):
    announce(f"sampler vocab {vocab}")
    rng = np.random.default_rng(vocab)
    rows = 7
    logits = rng.standard_normal((rows, vocab)) * 3
    if vocab > 4:
        logits[1, rng.integers(0, vocab, vocab // 3)] = -np.inf  # masked tokens
    temps = [0.3, 0.7, 1.0, 1.5, 2.0, 1e-12, 0.05]
    got = _run(logits, temps, seed=12345, offset=vocab, dev=dev)
    assert np.all((got >= 0) & (got < vocab))
    _check(got, logits, temps, 12345, vocab)
    if vocab > 4:
        assert np.isfinite(logits[1, got[1]])


def test_sampler_full_vocab(dev):
    # the decode batch: 256 rows over a 151936-token vocabulary
    announce("sampler 256 x 151936")
    rng = np.random.default_rng(7)
    rows, vocab = 256, 151936
    logits = (rng.standard_normal((rows, vocab)) * 2).astype(np.float32)
    temps = rng.uniform(0.5, 1.5, rows).astype(np.float32)
    got = _run(logits, temps, seed=2 ** 40 + 3, offset=17, dev=dev)
    _check(got, logits.astype(np.float64), temps, 2 ** 40 + 3, 17)


def test_sampler_frequencies(dev):
    announce("sampler frequencies")
    lg = np.array([1.0, 0.0, -0.5, 2.0, 0.3, -np.inf, 1.2, -1.0])
    rows = 40000
    for t in (0.5, 1.0, 2.0):
        got = _run(np.tile(lg, (rows, 1)), np.full(rows, t), seed=99, offset=int(t * 10), dev=dev)
        counts = np.bincount(got, minlength=len(lg))
        assert counts[5] == 0
        keep = np.isfinite(lg)
        expected = scipy.special.softmax(lg[keep] / t) * rows
        assert scipy.stats.chisquare(counts[keep], expected).pvalue > 1e-4, (t, counts)


def test_sampler_special_rows_and_streams(dev):
    announce("sampler special rows and streams")
    vocab = 1000
    lg = np.random.default_rng(3).standard_normal((6, vocab))
    lg[0] = -np.inf                 # nothing drawable: token 0
    lg[1, 123] = np.inf             # an infinite logit wins
    lg[2, [10, 20]] = np.inf        # ... the lowest index among ties
    lg[3, 500] += 80.0              # a dominant logit
    got = _run(lg, np.ones(6), 5, 0, dev)
    assert got[0] == 0 and got[1] == 123 and got[2] == 10 and got[3] == 500
    # same seed and offset -> same tokens; another offset -> new noise
    wide = np.random.default_rng(4).standard_normal((64, 5000))
    a = _run(wide, np.ones(64), 8, 1, dev)
    assert np.array_equal(a, _run(wide, np.ones(64), 8, 1, dev))
    b = _run(wide, np.ones(64), 8, 2, dev)
    assert (a != b).sum() > 32


def _run_strided(logits, temps, seed, offset, dev, pad):
    """logits [B, V] as the first V columns of a [B, V + pad] device tensor (rows V + pad elements apart)."""
    b, v = logits.shape
    wide = np.full((b, v + pad), 7.0, dtype=np.float32)  # the padding would win if it were read
    wide[:, :v] = logits
    lg = torch.as_tensor(wide).to(dev)[:, :v]
    assert lg.stride(0) == v + pad
    out = pa.pa_sample_gumbel(lg, torch.as_tensor(np.asarray(temps, np.float32)).to(dev), seed, offset)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("vocab,pad", [(12288, 4), (12288, 3), (20000, 8), (20000, 1)])
def test_sampler_strided_rows(dev, vocab, pad):
    # rows 16-byte aligned (pad a multiple of 4: vector loads) or not (single loads), padding never read
    announce(f"sampler strided rows vocab {vocab} pad {pad}")
    rng = np.random.default_rng(vocab + pad)
    logits = (rng.standard_normal((6, vocab)) * 2).astype(np.float32)
    temps = rng.uniform(0.5, 1.5, 6).astype(np.float32)
    got = _run_strided(logits, temps, 31, pad, dev, pad)
    assert np.all((got >= 0) & (got < vocab))
    _check(got, logits.astype(np.float64), temps, 31, pad)


def test_sampler_ties_across_layouts(dev):
    # +inf logits tie exactly: the lowest index must win wherever the tied elements sit (the same group of
    # three, neighbouring lanes, the end of one wave's 768-logit span and the start of the next, the
    # vector-loaded part against the row's ragged end)
    announce("sampler ties")
    vocab = 20000
    cases = [[9, 10, 11], [10, 11], [11, 12], [767, 768], [766, 1535, 1536], [12287, 12288],
             [18433, 19999], [19998, 19999], [5, 19999]]
    lg = np.random.default_rng(11).standard_normal((len(cases), vocab))
    for r, idx in enumerate(cases):
        lg[r, idx] = np.inf
    got = _run(lg, np.ones(len(cases)), 3, 4, dev)
    assert got.tolist() == [min(c) for c in cases]


@pytest.mark.parametrize("pad", [8, 1])
def test_sampler_batch_strided(dev, pad):
    # a decode-sized batch of 256 rows, 16-byte aligned with a ragged end (pad 8) or not aligned at all
    # (pad 1), with masked tokens; the padding never read
    announce(f"sampler 256 x 20000 pad {pad}")
    rng = np.random.default_rng(40 + pad)
    rows, vocab = 256, 20000
    logits = (rng.standard_normal((rows, vocab)) * 2).astype(np.float32)
    logits[::5, rng.integers(0, vocab, 3000)] = -np.inf
    temps = rng.uniform(0.3, 1.8, rows).astype(np.float32)
    got = _run_strided(logits, temps, 77, 9, dev, pad)
    assert np.all((got >= 0) & (got < vocab))
    _check(got, logits.astype(np.float64), temps, 77, 9)


def test_sampler_batch_ties_far_apart(dev):
    # exact ties in a 256-row batch over a 100003-token vocabulary: the lowest index wins across a wave's
    # 768-logit spans, across workgroups' 12288-logit chunks far apart in the row, and between the
    # vector-loaded part and the ragged end
    announce("sampler ties far apart")
    rows, vocab = 256, 100003
    cases = [[9, 10, 11], [767, 768], [12287, 12288], [49151, 49152], [1, 49152], [98303, 98304],
             [49152, 100002], [100001, 100002], [5, 100002], [60000, 20000]]
    lg = np.random.default_rng(12).standard_normal((rows, vocab)).astype(np.float32)
    for r in range(rows):
        lg[r, cases[r % len(cases)]] = np.inf
    got = _run(lg, np.ones(rows), 3, 4, dev)
    assert got.tolist() == [min(cases[r % len(cases)]) for r in range(rows)]
