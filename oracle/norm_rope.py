"""fp64 oracle of the step before the KV store: QK-RMSNorm and rotary embedding.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the HIP
library or its binding imports this module, and it imports nothing from them.

What it computes (page "nano-vLLM 最小化vLLM重新实现", section 6 "模型" and
"辅助层"): the model's attention layer takes the fused q/k/v projection of each
token, applies RMSNorm to every query head and every key head (QK-norm), then
the rotary position embedding with a precomputed cos/sin table, and the KV
store (section 5 "注意力机制") writes the rotated K and the untouched V into
the paged cache by slot.

Readings where the pages are silent (listed in the design doc):

* RMSNorm of a head vector x (length D) with weight w and epsilon eps is
  ``x / sqrt(mean(x**2) + eps) * w``; query heads share one weight vector,
  key heads another.
* Normalisation comes before the rotation.
* The rotation pairs dimension i with dimension i + D/2 (the two halves of
  the head vector) and turns each pair by the angle whose cosine and sine the
  table holds for the token's position: ``(a, b) -> (a cos - b sin,
  b cos + a sin)``, i.e. counter-clockwise.
* The table is an input: row p holds D/2 cosines then D/2 sines (fp32).
* The result is computed exactly (fp64) from the bf16 inputs and the fp32
  table; the kernel rounds once, to bf16, at the end.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import bf16_to_f64


def rms_norm(x, w, eps):
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * w (all fp64)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rotate_half_pairs(x, cos, sin):
    """Rotate pairs (i, i + D/2) of the last axis by the angles of cos/sin [..., D/2]."""
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * cos - b * sin, b * cos + a * sin], axis=-1)


def qk_norm_rope(qkv, positions, cos_sin, q_weight, k_weight, eps, num_q_heads, num_kv_heads):
    """Normalise and rotate the q and k heads of every token.

    qkv        uint16 bf16 bits [T, (Hq + 2 Hkv) * D]: q heads, then k heads,
               then v heads.
    positions  int [T], rows of cos_sin.
    cos_sin    float32 [max_position, D]: cos of the D/2 angles, then their sin.
    q_weight, k_weight  uint16 bf16 bits [D].
    Returns (q [T, Hq, D], k [T, Hkv, D]) in fp64 and v [T, Hkv, D] as bf16 bits.
    """
    qkv = np.asarray(qkv, dtype=np.uint16)
    t = qkv.shape[0]
    d = cos_sin.shape[1]
    h = d // 2
    heads = qkv.reshape(t, num_q_heads + 2 * num_kv_heads, d)
    q = bf16_to_f64(heads[:, :num_q_heads])
    k = bf16_to_f64(heads[:, num_q_heads:num_q_heads + num_kv_heads])
    v = heads[:, num_q_heads + num_kv_heads:].copy()
    table = np.asarray(cos_sin, dtype=np.float32).astype(np.float64)[np.asarray(positions, dtype=np.int64)]
    cos = table[:, None, :h]
    sin = table[:, None, h:]
    qn = rms_norm(q, bf16_to_f64(q_weight), eps)
    kn = rms_norm(k, bf16_to_f64(k_weight), eps)
    return rotate_half_pairs(qn, cos, sin), rotate_half_pairs(kn, cos, sin), v
