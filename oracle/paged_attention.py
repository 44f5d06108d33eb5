"""fp64 reference for the paged KV store, paged decode and varlen prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

Data conventions (shared with the C ABI only through these written rules, not
through code):

* bf16 values are carried as ``uint16`` bit patterns. The oracle widens them
  exactly (bits << 16 is the fp32 pattern; fp32 -> fp64 is exact).
* A per-layer cache is ``[num_blocks, block_size, num_kv_heads, head_dim]``
  (page "nano-vLLM 最小化vLLM重新实现", section 4 "模型运行器": one KV tensor
  ``[2, num_layers, num_blocks, block_size, num_kv_heads, head_dim]``; a layer's
  K and V caches are its two slices).
* A flat slot ``s`` names row ``s % block_size`` of physical block
  ``s // block_size``.

Readings where the pages are silent (each is listed in the design doc):

* grouped-query attention: query head ``h`` reads kv head ``h // G`` with
  ``G = num_q_heads // num_kv_heads`` (contiguous groups);
* a decode ``context_len`` counts the token just stored, so the query attends
  to positions ``0 .. L-1`` including itself; ``L == 0`` gives a zero row;
* causal prefill with fewer queries than keys aligns the queries with the last
  keys: query ``j`` of a sequence with ``nq`` queries and ``nk`` keys sits at
  position ``nk - nq + j`` and sees keys ``0 .. nk - nq + j``;
* a negative slot means "skip this token" (padding).
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    with np.errstate(invalid="ignore"):  # NaN patterns widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def slot_of(block_list, pos: int, block_size: int) -> int:
    """Flat cache slot of token position ``pos`` of a sequence.

    The sequence's block list maps logical block ``pos // block_size`` to a
    physical block; the token sits at row ``pos % block_size`` of it (page
    "nano-vLLM 最小化vLLM重新实现", section 3 "块管理器" and section 5 "注意力机制";
    page at hotelren.com/news/2273631, section 2.2, the per-sequence list of
    physical blocks used like a page table).
    """
    return int(block_list[pos // block_size]) * block_size + pos % block_size


def store_kvcache(k, v, slot_mapping, k_cache, v_cache):
    """Copy each token's K and V rows into the cache slot named by ``slot_mapping``.

    ``k``, ``v``: ``[T, Hkv, D]`` uint16; caches ``[NB, bs, Hkv, D]`` uint16.
    Returns new cache arrays; the inputs are not modified. Tokens whose slot is
    negative (padding) or past the last slot of the cache are skipped. Page
    "nano-vLLM 最小化vLLM重新实现", section 5 "注意力机制" (store kernel writing
    K/V into the paged cache by slot).
    """
    kc = np.array(k_cache, dtype=np.uint16, copy=True)
    vc = np.array(v_cache, dtype=np.uint16, copy=True)
    block_size = kc.shape[1]
    capacity = kc.shape[0] * block_size
    for t in range(len(slot_mapping)):
        s = int(slot_mapping[t])
        if s < 0 or s >= capacity:
            continue
        kc[s // block_size, s % block_size] = k[t]
        vc[s // block_size, s % block_size] = v[t]
    return kc, vc


def gather_rows(cache, block_list, n: int) -> np.ndarray:
    """Rows ``0 .. n-1`` of one sequence read through its block list: ``[n, Hkv, D]``.

    Only positions below ``n`` are touched, so whatever sits in the unused
    tail of the last block is never read.
    """
    block_size = cache.shape[1]
    rows = [cache[int(block_list[p // block_size]), p % block_size] for p in range(n)]
    if not rows:
        return np.zeros((0,) + cache.shape[2:], dtype=cache.dtype)
    return np.stack(rows)


def attention_rows(q, keys, values, scale: float, last_key) -> np.ndarray:
    """``softmax(scale * q kᵀ) v`` per query row, row ``j`` seeing keys ``0 .. last_key[j]``.

    ``q``: ``[m, D]``; ``keys``, ``values``: ``[n, D]`` (all fp64). A row whose
    ``last_key`` is negative sees no key and returns zeros. Page at
    bxzpzcl.cn/news/2159246, section 2.2.2 "两级注意力加速" (manual attention:
    scores ``q @ kᵀ / sqrt(head_dim)``, softmax over keys, times ``v``).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    m, n = q.shape[0], keys.shape[0]
    out = np.zeros((m, values.shape[1]), dtype=np.float64)
    if n == 0:
        return out
    scores = scale * (q @ keys.T)
    allowed = np.arange(n)[None, :] <= np.asarray(last_key)[:, None]
    for j in range(m):
        if not allowed[j].any():
            continue
        s = scores[j][allowed[j]]
        w = np.exp(s - s.max())
        out[j] = (w @ values[allowed[j]]) / w.sum()
    return out


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float) -> np.ndarray:
    """Paged decode attention: one query per sequence over its cached context.

    ``q``: ``[B, Hq, D]`` uint16; caches ``[NB, bs, Hkv, D]`` uint16;
    ``block_tables``: ``[B, W]`` int; ``context_lens``: ``[B]``. Returns
    ``[B, Hq, D]`` fp64. Page "nano-vLLM 最小化vLLM重新实现", section 5
    "注意力机制" (decode attention over the paged KV cache).
    """
    n_seq, hq, d = q.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    out = np.zeros((n_seq, hq, d), dtype=np.float64)
    for b in range(n_seq):
        length = int(context_lens[b])
        if length == 0:
            continue
        keys = bf16_to_f64(gather_rows(k_cache, block_tables[b], length))
        values = bf16_to_f64(gather_rows(v_cache, block_tables[b], length))
        qb = bf16_to_f64(q[b])
        for h in range(hq):
            g = h // group
            out[b, h] = attention_rows(qb[h][None, :], keys[:, g], values[:, g], scale,
                                       [length - 1])[0]
    return out


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale: float, causal: bool = True,
                   block_table=None) -> np.ndarray:
    """Varlen prefill attention over packed sequences.

    ``q``: ``[Tq, Hq, D]`` uint16 packed by ``cu_seqlens_q``. Without a block
    table, ``k`` and ``v`` are packed ``[Tk, Hkv, D]`` arrays split by
    ``cu_seqlens_k``; with one, they are the paged caches and sequence ``i``
    reads its ``nk`` keys through ``block_table[i]`` (prefix-cached blocks
    included). Returns ``[Tq, Hq, D]`` fp64. Page "nano-vLLM 最小化vLLM重新实现",
    section 5 "注意力机制" (varlen prefill with an optional block table for the
    prefix cache); page at hotelren.com/news/2273631, section 4.4 (prefix
    caching: the shared prefix's KV is reused, only the remainder is computed).
    """
    tq, hq, d = q.shape
    hkv = k.shape[-2]
    group = hq // hkv
    out = np.zeros((tq, hq, d), dtype=np.float64)
    for i in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[i]), int(cu_seqlens_q[i + 1])
        k0, k1 = int(cu_seqlens_k[i]), int(cu_seqlens_k[i + 1])
        nq, nk = q1 - q0, k1 - k0
        if nq == 0:
            continue
        if block_table is None:
            keys = bf16_to_f64(k[k0:k1])
            values = bf16_to_f64(v[k0:k1])
        else:
            keys = bf16_to_f64(gather_rows(k, block_table[i], nk))
            values = bf16_to_f64(gather_rows(v, block_table[i], nk))
        if causal:
            last_key = [nk - nq + j for j in range(nq)]
        else:
            last_key = [nk - 1] * nq
        qi = bf16_to_f64(q[q0:q1])
        for h in range(hq):
            g = h // group
            out[q0:q1, h] = attention_rows(qi[:, h], keys[:, g], values[:, g], scale, last_key)
    return out

