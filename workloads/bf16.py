"""bf16 encoding of synthetic inputs (bit patterns carried as uint16).

Input encoding only: this module rounds generated fp32/fp64 values to bf16 with
round-to-nearest-even and nothing else. It holds no attention, paging or store
arithmetic.
"""

from __future__ import annotations

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def encode(x) -> np.ndarray:
    """Round to bf16 (RNE, via fp32) and return the uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def decode_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0, 1) samples rounded to bf16 bit patterns."""
    return encode(rng.standard_normal(shape, dtype=np.float32))
