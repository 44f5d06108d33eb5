"""Rotary-embedding cos/sin table and norm weights: inputs of the fused QK-norm + RoPE + store.

Input construction only. The fused operation takes the table as given (the
model precomputes it once; page "nano-vLLM 最小化vLLM重新实现", "辅助层":
RotaryEmbedding keeps a precomputed cos/sin cache), so neither the kernel nor
the oracle computes angles. The table here follows the usual frequency
schedule theta_i = base ** (-2 i / D), i < D/2, with the base a parameter
(the pages do not give one): row p = [cos(p theta_0 ..), sin(p theta_0 ..)],
computed in fp64 and stored as fp32.
"""

from __future__ import annotations

import numpy as np

from .bf16 import encode


def cos_sin_table(max_position: int, head_dim: int, base: float = 1.0e6) -> np.ndarray:
    """float32 [max_position, head_dim]: cosines of the head_dim/2 angles, then sines."""
    half = head_dim // 2
    inv_freq = base ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = np.arange(max_position, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def norm_weight(rng: np.random.Generator, head_dim: int) -> np.ndarray:
    """bf16 bits of an RMSNorm weight around 1 (1 + 0.1 N(0, 1))."""
    return encode(1.0 + 0.1 * rng.standard_normal(head_dim))
