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
  its published definition, Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011): element i of row b
  takes field i % 6 of the block at counter (i // 6, b, offset mod 2^32,
  offset // 2^32) under key (seed mod 2^32, seed // 2^32). A block's four
  32-bit words w0..w3 form two 64-bit values X0 = w1 * 2^32 + w0 and
  X1 = w3 * 2^32 + w2; fields 0, 1, 2 are bits 63..43, 42..22 and 21..1 of X0,
  fields 3, 4, 5 the same bits of X1. A field w gives u = (w + 1/2) / 2^21 in
  (0, 1) (exact in fp32: w + 1/2 has 22 significant bits) and E = -ln(u).
  Philox4x32's multiplies are 32 x 32 bits, so a block of six 21-bit fields
  costs 20 of them.
* Ties go to the lowest index; temperatures at or below 1e-10 are raised to
  1e-10.
"""

from __future__ import annotations

import numpy as np

M0, M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
W0, W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)
MIN_TEMPERATURE = 1e-10
FIELDS_PER_BLOCK = 6


def philox4x32(counter, key):
    """Philox4x32-10 blocks: counter [..., 4], key [..., 2] of 32-bit values (any integer dtype) ->
    uint64 [..., 4] holding the four 32-bit output words."""
    x = [np.asarray(counter[..., i], dtype=np.uint64) & _LO32 for i in range(4)]
    k0 = np.asarray(key[..., 0], dtype=np.uint64) & _LO32
    k1 = np.asarray(key[..., 1], dtype=np.uint64) & _LO32
    for _ in range(10):
        p0 = M0 * x[0]  # 32 x 32 bits: exact in uint64
        p1 = M1 * x[2]
        x = [(p1 >> _S32) ^ x[1] ^ k0, p1 & _LO32, (p0 >> _S32) ^ x[3] ^ k1, p0 & _LO32]
        k0 = (k0 + W0) & _LO32
        k1 = (k1 + W1) & _LO32
    return np.stack(x, axis=-1)


def uniforms(num_rows: int, vocab_size: int, seed: int, offset: int) -> np.ndarray:
    """u[b, i] in (0, 1) for every element (fp64; each value is exact in fp32)."""
    nblk = -(-vocab_size // FIELDS_PER_BLOCK)
    j, b = np.meshgrid(np.arange(nblk, dtype=np.uint64), np.arange(num_rows, dtype=np.uint64))
    off, sd = int(offset) % 2 ** 64, int(seed) % 2 ** 64
    ctr = np.stack([j, b, np.full_like(j, np.uint64(off % 2 ** 32)), np.full_like(j, np.uint64(off >> 32))],
                   axis=-1)
    key = np.empty(ctr.shape[:-1] + (2,), dtype=np.uint64)
    key[..., 0] = np.uint64(sd % 2 ** 32)
    key[..., 1] = np.uint64(sd >> 32)
    w = philox4x32(ctr, key)
    halves = [(w[..., 1] << _S32) | w[..., 0], (w[..., 3] << _S32) | w[..., 2]]
    mask = np.uint64(0x1FFFFF)
    fields = np.empty((num_rows, nblk, FIELDS_PER_BLOCK), dtype=np.uint64)
    for h, x in enumerate(halves):
        fields[..., 3 * h] = x >> np.uint64(43)
        fields[..., 3 * h + 1] = (x >> np.uint64(22)) & mask
        fields[..., 3 * h + 2] = (x >> np.uint64(1)) & mask
    fields = fields.reshape(num_rows, nblk * FIELDS_PER_BLOCK)
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
