"""Seeded N(0, 1) bf16 values for a Workload, materialised with torch on a device.

Input generation only: fp32 normals from a seeded torch generator, rounded to
bf16 (round to nearest even), laid out as the kernels receive them:

* q, k and v are column slices of one fused [T, (Hq + 2 Hkv) * D] projection
  output, so K/V reach the store as strided views (page "nano-vLLM
  最小化vLLM重新实现", section 4 "模型运行器": q/k/v are packed into one qkv_proj);
* each cache is [num_blocks, block_size, Hkv, D]; every row that holds no
  token is filled with bf16 NaN (0x7FC0), standing in for the stale contents
  of reused blocks, so that any read of such a row shows up in the output;
* rows a sequence already holds before the store (decode positions
  0 .. L-2, the shared prefix of a prefix-cached batch) get N(0, 1) values.

Values differ between devices for the same seed (each device has its own
generator); every consumer reads the one materialised copy.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import Workload

BF16_NAN_BITS = 0x7FC0


def _generator(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + stream)
    return g


def normal_bf16(shape, gen: torch.Generator, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def nan_bf16(shape, device) -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.bfloat16, device=device)
    t.view(torch.int16).fill_(BF16_NAN_BITS)
    return t


def to_u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 numpy bit patterns on the host."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Batch:
    wl: Workload
    qkv: torch.Tensor          # [T, (Hq + 2 Hkv) * D] fused projection output
    q: torch.Tensor            # [T, Hq, D] view
    k_new: torch.Tensor        # [T, Hkv, D] strided view
    v_new: torch.Tensor        # [T, Hkv, D] strided view
    k_cache: torch.Tensor      # [NB, bs, Hkv, D]
    v_cache: torch.Tensor
    block_tables: torch.Tensor   # int32 [S, W]
    slot_mapping: torch.Tensor   # int32 [T]
    context_lens: torch.Tensor | None = None  # int32 [S] (decode)
    cu_seqlens_q: torch.Tensor | None = None  # int32 [S + 1] (prefill)
    cu_seqlens_k: torch.Tensor | None = None


def _fill_rows(cache: torch.Tensor, wl: Workload, gen, device, chunk_blocks: int = 1024) -> None:
    """Give N(0,1) values to the rows each sequence holds before the store."""
    bs = wl.block_size
    items = []  # (physical block, valid rows)
    seen = set()
    for s in range(wl.num_seqs):
        pre = int(wl.pre_len[s])
        for i in range(-(-pre // bs)):
            blk = int(wl.block_tables[s, i])
            if blk in seen:  # a shared prefix block is filled once
                continue
            seen.add(blk)
            items.append((blk, min(bs, pre - i * bs)))
    if not items:
        return
    blocks = torch.tensor([b for b, _ in items], dtype=torch.int64, device=device)
    rows = torch.tensor([r for _, r in items], dtype=torch.int64, device=device)
    shape = cache.shape[1:]
    for c0 in range(0, len(items), chunk_blocks):
        c1 = min(len(items), c0 + chunk_blocks)
        vals = normal_bf16((c1 - c0,) + tuple(shape), gen, device)
        keep = torch.arange(bs, device=device)[None, :] < rows[c0:c1, None]
        vals.view(torch.int16)[~keep] = BF16_NAN_BITS
        cache[blocks[c0:c1]] = vals


def materialize(wl: Workload, device, fill_nan: bool = True) -> Batch:
    """All tensors of a workload on `device` (values seeded by wl.seed)."""
    hq, hkv, d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    t = wl.num_tokens if wl.kind == "prefill" else wl.num_seqs
    gen = _generator(device, wl.seed, 10)
    qkv = normal_bf16((t, (hq + 2 * hkv) * d), gen, device)
    q = qkv[:, : hq * d].view(t, hq, d)
    k_new = qkv[:, hq * d:(hq + hkv) * d].unflatten(1, (hkv, d))
    v_new = qkv[:, (hq + hkv) * d:].unflatten(1, (hkv, d))
    shape = (wl.num_blocks, wl.block_size, hkv, d)
    if fill_nan:
        k_cache, v_cache = nan_bf16(shape, device), nan_bf16(shape, device)
    else:
        k_cache = torch.zeros(shape, dtype=torch.bfloat16, device=device)
        v_cache = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    _fill_rows(k_cache, wl, _generator(device, wl.seed, 11), device)
    _fill_rows(v_cache, wl, _generator(device, wl.seed, 12), device)
    i32 = lambda a: torch.as_tensor(np.ascontiguousarray(a), dtype=torch.int32).to(device)  # noqa: E731
    batch = Batch(wl, qkv, q, k_new, v_new, k_cache, v_cache, i32(wl.block_tables), i32(wl.slot_mapping))
    if wl.kind == "decode":
        # decode stores the new token of every sequence with L >= 1; k_new/v_new
        # rows are indexed by sequence, so pad the slot list to one per sequence
        slots = np.full(wl.num_seqs, -1, dtype=np.int32)
        slots[wl.store_seq] = wl.slot_mapping
        batch.slot_mapping = i32(slots)
        batch.context_lens = i32(wl.context_lens)
    else:
        batch.cu_seqlens_q = i32(wl.cu_seqlens_q)
        batch.cu_seqlens_k = i32(wl.cu_seqlens_k)
    return batch
