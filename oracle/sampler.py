"""fp64 oracle of the Gumbel-max sampler: exponential noise, then an argmax.

TEST INFRASTRUCTURE ONLY (see the package docstring); it shares no code with
the HIP sampler.

What it computes (page "nano-vLLM 最小化vLLM重新实现", "辅助层": the sampler
uses the Gumbel-max trick, exponential noise followed by an argmax; "关键设计
选择": greedy sampling is not allowed, temperatures are above 1e-10): for row b
with logits l and temperature T,

    token_b = argmax_i softmax(l / T)_i / E_i,   E_i ~ Exp(1) independent,

which draws token i with probability softmax(l / T)_i.

Readings (listed in the design doc):

* The noise is drawn by a counter-based generator both sides implement from
  its published definition, Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011): element i of row b
  takes a 21-bit field of 64-bit word (i // 3) % 4 of the block at counter
  (i // 12, b, offset, 0) under key (seed, 0) -- bits 63..43 for i % 3 == 0,
  42..22 for i % 3 == 1, 21..1 for i % 3 == 2 -- and w gives
  u = (w + 1/2) / 2^21 in (0, 1) (exact in fp32: w + 1/2 has 22 significant
  bits) and E = -ln(u). Three fields per word cut the generator's cost per
  element to a third of a one-field-per-word layout.
* Ties go to the lowest index; temperatures at or below 1e-10 are raised to
  1e-10.
"""

from __future__ import annotations

import numpy as np

M0, M1 = np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157)
W0, W1 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)
MIN_TEMPERATURE = 1e-10


def _mulhilo(a, b):
    """Full 64 x 64 -> 128-bit product of uint64 arrays: (hi, lo)."""
    a0, a1 = a & _LO32, a >> _S32
    b0, b1 = b & _LO32, b >> _S32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = (p00 & _LO32) | ((mid & _LO32) << _S32)
    return hi, lo


def philox4x64(counter, key):
    """Philox4x64-10 blocks: counter uint64 [..., 4], key uint64 [..., 2] -> uint64 [..., 4]."""
    x = [np.asarray(counter[..., i], dtype=np.uint64) for i in range(4)]
    k0 = np.asarray(key[..., 0], dtype=np.uint64)
    k1 = np.asarray(key[..., 1], dtype=np.uint64)
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo(M0, x[0])
            hi1, lo1 = _mulhilo(M1, x[2])
            x = [hi1 ^ x[1] ^ k0, lo1, hi0 ^ x[3] ^ k1, lo0]
            k0 = k0 + W0
            k1 = k1 + W1
    return np.stack(x, axis=-1)


def uniforms(num_rows: int, vocab_size: int, seed: int, offset: int) -> np.ndarray:
    """u[b, i] in (0, 1) for every element (fp64; each value is exact in fp32)."""
    nblk = -(-vocab_size // 12)
    j, b = np.meshgrid(np.arange(nblk, dtype=np.uint64), np.arange(num_rows, dtype=np.uint64))
    ctr = np.stack([j, b, np.full_like(j, np.uint64(offset)), np.zeros_like(j)], axis=-1)
    key = np.zeros(ctr.shape[:-1] + (2,), dtype=np.uint64)
    key[..., 0] = np.uint64(seed)
    words = philox4x64(ctr, key).reshape(num_rows, nblk * 4)
    mask = np.uint64(0x1FFFFF)
    fields = np.empty((num_rows, nblk * 12), dtype=np.uint64)
    fields[:, 0::3] = words >> np.uint64(43)
    fields[:, 1::3] = (words >> np.uint64(22)) & mask
    fields[:, 2::3] = (words >> np.uint64(1)) & mask
    return (fields[:, :vocab_size].astype(np.float64) + 0.5) / 2.0 ** 21


def scores(logits, temperatures, seed: int, offset: int) -> np.ndarray:
    """log(softmax(l / T)_i / E_i) up to a per-row constant: l_i / T - ln(-ln u_i) (fp64)."""
    lg = np.asarray(logits, dtype=np.float64)
    t = np.maximum(np.asarray(temperatures, dtype=np.float64), MIN_TEMPERATURE)
    u = uniforms(lg.shape[0], lg.shape[1], seed, offset)
    e = -np.log(u)
    with np.errstate(invalid="ignore"):
        return lg / t[:, None] - np.log(e)


def sample(logits, temperatures, seed: int, offset: int) -> np.ndarray:
    """int64 [B]: argmax_i softmax(l / T)_i / E_i (lowest index on ties)."""
    return np.argmax(scores(logits, temperatures, seed, offset), axis=1)
