"""Python binding of libpa.so, the paged-KV-cache attention library for MI355X.

Argument marshalling only: every function passes tensor addresses, strides and
sizes to the C entry point of the same name in include/pa.h, on the current
HIP stream, and raises PAError if it returns a non-zero status. All compute
runs in the library's HIP kernels; there is no fallback path.

Tensors are torch tensors on the GPU: bf16 data, int32 metadata.
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import LibraryMissing  # noqa: F401

__all__ = [
    "PAError", "LibraryMissing", "pa_store_kvcache", "pa_qk_norm_rope_store", "pa_decode", "pa_store_decode",
    "pa_decode_workspace_size", "pa_decode_split_waves", "pa_prefill_varlen", "pa_status_string", "pa_last_error", "pa_version",
    "library_path", "DecodeGraphs", "pa_sample_gumbel", "pa_sample_workspace_size", "pa_store_decode_noalloc",
    "pa_store_prefill_varlen",
]


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _lib.load()
        self.status = status
        msg = lib.pa_last_error().decode() or lib.pa_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({lib.pa_status_string(status).decode()}): {msg}")


def library_path() -> str:
    return _lib.LIB_PATH


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise PAError(fn, status)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


_BF16, _I32, _F32, _U8 = torch.bfloat16, torch.int32, torch.float32, torch.uint8


def _want(t, name: str, dtype, dim=None, contiguous=False, optional=False) -> None:
    """Check a tensor argument before its address crosses the C ABI (which sees only pointers).

    Raises TypeError for a non-tensor or a wrong dtype and ValueError for a wrong rank or a
    required but missing contiguity. Shapes across arguments are checked next (_shape), and
    the device last (_device), so every shape mismatch is reported even for host tensors.
    """
    if t is None:
        if optional:
            return
        raise TypeError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(t, name: str, want) -> None:
    """ValueError unless t (if given) has shape `want`; None in `want` matches any extent."""
    if t is None:
        return
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and int(w) != g for g, w in zip(got, want)):
        shown = tuple("*" if w is None else int(w) for w in want)
        raise ValueError(f"{name} must have shape {shown}, got {got}")


def _device(**tensors) -> torch.device:
    """The one GPU all given tensors sit on; ValueError for a host tensor or a mix of devices."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU, got {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
    return dev


def _stream(stream, device) -> int:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(device).cuda_stream


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a [rows, heads, dims] view whose heads x dims are contiguous."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be [rows, heads, dims] with contiguous heads x dims, got "
                         f"shape {tuple(t.shape)} strides {t.stride()}")
    return t.stride(0)


def pa_status_string(status: int) -> str:
    return _lib.load().pa_status_string(status).decode()


def pa_last_error() -> str:
    return _lib.load().pa_last_error().decode()


def pa_version() -> int:
    return _lib.load().pa_version()


def pa_store_kvcache(k, v, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write k[t] / v[t] ([T, Hkv, D] bf16) into the caches ([NB, bs, Hkv, D]) at slot_mapping[t]."""
    _want(k_cache, "k_cache", _BF16, 4, True)
    _want(v_cache, "v_cache", _BF16, 4, True)
    _want(k, "k", _BF16, 3)
    _want(v, "v", _BF16, 3)
    _want(slot_mapping, "slot_mapping", _I32, 1, True)
    nb, bs, hkv, d = k_cache.shape
    t = int(slot_mapping.shape[0])
    _shape(v_cache, "v_cache", k_cache.shape)
    _shape(k, "k", (t, hkv, d))
    _shape(v, "v", (t, hkv, d))
    dev = _device(k_cache=k_cache, v_cache=v_cache, k=k, v=v, slot_mapping=slot_mapping)
    lib = _lib.load()
    _check("pa_store_kvcache", lib.pa_store_kvcache(
        _ptr(k), _rows(k, "k"), _ptr(v), _rows(v, "v"), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
        t, hkv, d, nb, bs, _stream(stream, dev)))


def pa_qk_norm_rope_store(qkv, q_norm_weight, k_norm_weight, eps: float, cos_sin, positions, k_cache, v_cache,
                          slot_mapping, num_q_heads: int, q_out=None, stream=None):
    """QK-RMSNorm + rotary embedding of qkv [T, (Hq + 2 Hkv) * D] bf16, then the KV store.

    cos_sin: [max_position, D] fp32 (cosines, then sines); positions, slot_mapping: [T] int32.
    Returns q_out [T, Hq, D] bf16 (allocated when not given; may be a view of qkv's q columns).
    """
    _want(qkv, "qkv", _BF16, 2)
    for name, x in (("k_cache", k_cache), ("v_cache", v_cache)):
        _want(x, name, _BF16, 4, True)
    for name, x in (("q_norm_weight", q_norm_weight), ("k_norm_weight", k_norm_weight)):
        _want(x, name, _BF16, 1, True)
    _want(cos_sin, "cos_sin", _F32, 2, True)
    _want(positions, "positions", _I32, 1, True)
    _want(slot_mapping, "slot_mapping", _I32, 1, True)
    _want(q_out, "q_out", _BF16, 3, optional=True)
    nb, bs, hkv, d = k_cache.shape
    t, hq = int(qkv.shape[0]), int(num_q_heads)
    _shape(v_cache, "v_cache", k_cache.shape)
    _shape(qkv, "qkv", (t, (hq + 2 * hkv) * d))
    _shape(q_norm_weight, "q_norm_weight", (d,))
    _shape(k_norm_weight, "k_norm_weight", (d,))
    _shape(cos_sin, "cos_sin", (None, d))
    _shape(positions, "positions", (t,))
    _shape(slot_mapping, "slot_mapping", (t,))
    _shape(q_out, "q_out", (t, hq, d))
    if qkv.stride(1) != 1:
        raise ValueError(f"qkv must be [T, (Hq + 2 Hkv) * D] with contiguous columns, got strides {qkv.stride()}")
    dev = _device(qkv=qkv, k_cache=k_cache, v_cache=v_cache, q_norm_weight=q_norm_weight,
                  k_norm_weight=k_norm_weight, cos_sin=cos_sin, positions=positions, slot_mapping=slot_mapping,
                  q_out=q_out)
    lib = _lib.load()
    if q_out is None:
        q_out = torch.empty((t, hq, d), dtype=torch.bfloat16, device=dev)
    _check("pa_qk_norm_rope_store", lib.pa_qk_norm_rope_store(
        _ptr(q_out), _rows(q_out, "q_out"), _ptr(qkv), qkv.stride(0), _ptr(q_norm_weight), _ptr(k_norm_weight),
        float(eps), _ptr(cos_sin), int(cos_sin.shape[0]), _ptr(positions), _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), t, hq, hkv, d, nb, bs, _stream(stream, dev)))
    return q_out


def pa_sample_workspace_size(num_rows: int, vocab_size: int) -> int:
    return int(_lib.load().pa_sample_workspace_size(num_rows, vocab_size))


def pa_sample_gumbel(logits, temperatures, seed: int, offset: int, tokens=None, workspace=None, stream=None):
    """One token per row of logits [B, V] fp32 (temperatures [B] fp32): int32 [B]."""
    _want(logits, "logits", _F32, 2)
    _want(temperatures, "temperatures", _F32, 1, True)
    _want(tokens, "tokens", _I32, 1, True, optional=True)
    _want(workspace, "workspace", _U8, 1, True, optional=True)
    b, v = int(logits.shape[0]), int(logits.shape[1])
    _shape(temperatures, "temperatures", (b,))
    _shape(tokens, "tokens", (b,))
    if logits.stride(1) != 1:
        raise ValueError("logits must be [rows, vocab] with contiguous rows")
    dev = _device(logits=logits, temperatures=temperatures, tokens=tokens, workspace=workspace)
    lib = _lib.load()
    if tokens is None:
        tokens = torch.empty(b, dtype=torch.int32, device=dev)
    need = lib.pa_sample_workspace_size(b, v)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check("pa_sample_gumbel", lib.pa_sample_gumbel(
        _ptr(tokens), _ptr(logits), logits.stride(0), _ptr(temperatures), b, v, int(seed) & (2 ** 64 - 1),
        int(offset) & (2 ** 64 - 1), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, dev)))
    return tokens


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                             split_waves=0) -> int:
    return int(_lib.load().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                    max_context_len, split_waves))


def pa_decode_split_waves(num_seqs, num_q_heads, num_kv_heads, max_context_len, split_waves=0) -> int:
    return int(_lib.load().pa_decode_split_waves(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                                 split_waves))


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, out, workspace, k_new=None, v_new=None,
                 need_new=False, batch=None):
    """Checks shared by the decode entry points: dtypes and ranks, then every shape against
    q [B, Hq, D] and the cache [NB, bs, Hkv, D] (batch: the rows the buffers must hold, B by
    default), then the device. Returns the device."""
    _want(q, "q", _BF16, 3)
    _want(k_cache, "k_cache", _BF16, 4, True)
    _want(v_cache, "v_cache", _BF16, 4, True)
    _want(block_tables, "block_tables", _I32, 2, True)
    _want(context_lens, "context_lens", _I32, 1, True)
    _want(out, "out", _BF16, 3, True, optional=True)
    _want(workspace, "workspace", _U8, 1, True, optional=True)
    _want(k_new, "k_new", _BF16, 3, optional=not need_new)
    _want(v_new, "v_new", _BF16, 3, optional=not need_new)
    b, hq, d = (int(x) for x in q.shape)
    b = b if batch is None else int(batch)
    _shape(q, "q", (b, hq, d))
    _shape(v_cache, "v_cache", k_cache.shape)
    _shape(k_cache, "k_cache", (None, None, None, d))
    hkv = int(k_cache.shape[2])
    _shape(block_tables, "block_tables", (b, None))
    _shape(context_lens, "context_lens", (b,))
    _shape(out, "out", (b, hq, d))
    _shape(k_new, "k_new", (b, hkv, d))
    _shape(v_new, "v_new", (b, hkv, d))
    return _device(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables, context_lens=context_lens,
                   out=out, workspace=workspace, k_new=k_new, v_new=v_new)


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, max_context_len: int, out=None,
              workspace=None, split_waves: int = 0, stream=None):
    """Paged decode: q [B, Hq, D] bf16 -> out [B, Hq, D] bf16.

    workspace: a uint8 device tensor of at least pa_decode_workspace_size(...)
    bytes; allocated here when not given.
    """
    dev = _decode_args(q, k_cache, v_cache, block_tables, context_lens, out, workspace)
    lib = _lib.load()
    b, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.bfloat16, device=dev)
    need = lib.pa_decode_workspace_size(b, hq, hkv, d, max_context_len, split_waves)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode", lib.pa_decode(
        _ptr(out), _ptr(q), _rows(q, "q"), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(context_lens), b, hq, hkv, d, bs, int(max_context_len), float(scale),
        int(split_waves), _ptr(workspace), ws_bytes, _stream(stream, dev)))
    return out


def pa_store_decode(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale: float,
                    max_context_len: int, out=None, workspace=None, split_waves: int = 0, stream=None):
    """Store each sequence's new token at position L - 1 (through its block table), then paged decode:
    q [B, Hq, D], k_new / v_new [B, Hkv, D] bf16 -> out [B, Hq, D] bf16.

    Two kernels: the split kernel reads the new token's K/V from k_new / v_new, and the finalize
    kernel, which runs after it, writes them into the cache at position L - 1.
    workspace: as for pa_decode (allocated here when not given).
    """
    dev = _decode_args(q, k_cache, v_cache, block_tables, context_lens, out, workspace, k_new, v_new, True)
    lib = _lib.load()
    b, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.bfloat16, device=dev)
    need = lib.pa_decode_workspace_size(b, hq, hkv, d, max_context_len, split_waves)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_store_decode", lib.pa_store_decode(
        _ptr(out), _ptr(q), _rows(q, "q"), _ptr(k_new), _rows(k_new, "k_new"), _ptr(v_new), _rows(v_new, "v_new"),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), b, hq,
        hkv, d, bs, int(max_context_len), float(scale), int(split_waves), _ptr(workspace), ws_bytes,
        _stream(stream, dev)))
    return out


def pa_store_decode_noalloc(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale: float,
                            max_context_len: int, out, split_waves: int = 0, stream=None):
    """pa_store_decode with the library's static scratch as the workspace: allocates nothing, so
    `out` ([B, Hq, D] bf16) is required. Calls that overlap on one GPU race on the scratch."""
    if out is None:
        raise TypeError("out is required (this entry point allocates nothing)")
    dev = _decode_args(q, k_cache, v_cache, block_tables, context_lens, out, None, k_new, v_new, True)
    lib = _lib.load()
    b, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    _check("pa_store_decode_noalloc", lib.pa_store_decode_noalloc(
        _ptr(out), _ptr(q), _rows(q, "q"), _ptr(k_new), _rows(k_new, "k_new"), _ptr(v_new), _rows(v_new, "v_new"),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), b, hq,
        hkv, d, bs, int(max_context_len), float(scale), int(split_waves), _stream(stream, dev)))
    return out


def pa_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, scale: float,
                      causal: bool = True, block_table=None, out=None, stream=None):
    """Varlen prefill: q [Tq, Hq, D] bf16 -> out [Tq, Hq, D] bf16.

    Without block_table, k / v are packed [Tk, Hkv, D] (row strides may exceed
    Hkv * D); with it, k / v are the caches [NB, bs, Hkv, D].
    """
    _want(q, "q", _BF16, 3)
    kdim = 3 if block_table is None else 4
    _want(k, "k", _BF16, kdim, block_table is not None)
    _want(v, "v", _BF16, kdim, block_table is not None)
    _want(cu_seqlens_q, "cu_seqlens_q", _I32, 1, True)
    _want(cu_seqlens_k, "cu_seqlens_k", _I32, 1, True)
    _want(block_table, "block_table", _I32, 2, True, optional=True)
    _want(out, "out", _BF16, 3, True, optional=True)
    tq, hq, d = (int(x) for x in q.shape)
    num_seqs = int(cu_seqlens_q.shape[0]) - 1
    if num_seqs < 0:
        raise ValueError("cu_seqlens_q must hold num_seqs + 1 >= 1 offsets")
    _shape(cu_seqlens_k, "cu_seqlens_k", cu_seqlens_q.shape)
    _shape(out, "out", q.shape)
    _shape(v, "v", k.shape)
    _shape(k, "k", (None,) * (kdim - 1) + (d,))
    _shape(block_table, "block_table", (num_seqs, None))
    dev = _device(q=q, k=k, v=v, cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, block_table=block_table,
                  out=out)
    lib = _lib.load()
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.bfloat16, device=dev)
    if block_table is None:
        hkv = int(k.shape[1])
        ks, vs, width, bs = _rows(k, "k"), _rows(v, "v"), 0, 0
    else:
        _, bs, hkv, _ = (int(x) for x in k.shape)
        ks, vs, width = hkv * d, hkv * d, int(block_table.shape[1])
    _check("pa_prefill_varlen", lib.pa_prefill_varlen(
        _ptr(out), _ptr(q), _rows(q, "q"), _ptr(k), _ptr(v), ks, vs, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        num_seqs, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, float(scale), 1 if causal else 0,
        _ptr(block_table), width, bs, _stream(stream, dev)))
    return out


def pa_store_prefill_varlen(q, k_new, v_new, k_cache, v_cache, slot_mapping, cu_seqlens_q, cu_seqlens_k,
                            max_seqlen_q: int, max_seqlen_k: int, scale: float, causal: bool = True, block_table=None,
                            out=None, stream=None):
    """Store the new tokens (k_new / v_new [Tq, Hkv, D], one per query, at slot_mapping [Tq]) and run the
    varlen prefill in one call: q [Tq, Hq, D] -> out [Tq, Hq, D] bf16. Without block_table every key is
    new (nk == nq); with it, keys before the new tokens come from the caches through the table."""
    _want(q, "q", _BF16, 3)
    _want(k_new, "k_new", _BF16, 3)
    _want(v_new, "v_new", _BF16, 3)
    _want(k_cache, "k_cache", _BF16, 4, True)
    _want(v_cache, "v_cache", _BF16, 4, True)
    _want(slot_mapping, "slot_mapping", _I32, 1, True)
    _want(cu_seqlens_q, "cu_seqlens_q", _I32, 1, True)
    _want(cu_seqlens_k, "cu_seqlens_k", _I32, 1, True)
    _want(block_table, "block_table", _I32, 2, True, optional=True)
    _want(out, "out", _BF16, 3, True, optional=True)
    tq, hq, d = (int(x) for x in q.shape)
    nb, bs, hkv, _ = (int(x) for x in k_cache.shape)
    num_seqs = int(cu_seqlens_q.shape[0]) - 1
    if num_seqs < 0:
        raise ValueError("cu_seqlens_q must hold num_seqs + 1 >= 1 offsets")
    _shape(v_cache, "v_cache", k_cache.shape)
    _shape(k_cache, "k_cache", (None, None, None, d))
    _shape(k_new, "k_new", (tq, hkv, d))
    _shape(v_new, "v_new", (tq, hkv, d))
    _shape(slot_mapping, "slot_mapping", (tq,))
    _shape(cu_seqlens_k, "cu_seqlens_k", cu_seqlens_q.shape)
    _shape(block_table, "block_table", (num_seqs, None))
    _shape(out, "out", q.shape)
    dev = _device(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, slot_mapping=slot_mapping,
                  cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k, block_table=block_table, out=out)
    lib = _lib.load()
    if out is None:
        out = torch.empty((tq, hq, d), dtype=torch.bfloat16, device=dev)
    width = 0 if block_table is None else int(block_table.shape[1])
    _check("pa_store_prefill_varlen", lib.pa_store_prefill_varlen(
        _ptr(out), _ptr(q), _rows(q, "q"), _ptr(k_new), _rows(k_new, "k_new"), _ptr(v_new), _rows(v_new, "v_new"),
        _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), num_seqs,
        int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, float(scale), 1 if causal else 0, _ptr(block_table), width,
        bs, nb, _stream(stream, dev)))
    return out


class DecodeGraphs:
    """Graph-captured decode steps (pa_decode_graphs_*): pa_store_decode captured once per batch size.

    The tensors are the step's fixed device buffers, sized for max(batch_sizes): q [B, Hq, D],
    k_new / v_new [B, Hkv, D] views, block_tables [B, W], context_lens [B] (int32), out [B, Hq, D],
    workspace (uint8, >= pa_decode_workspace_size for the largest batch). The binding also holds
    `live_batch`, a one-element int32 device tensor. For each step fill rows 0 .. batch - 1 and write
    batch to live_batch (or let launch() write it), then launch(batch): one graph launch; rows past
    batch are empty contexts (zero output rows, nothing stored, not read).
    Capture needs a stream other than the legacy default stream (stream or the current torch stream).
    """

    def __init__(self, q, k_new, v_new, block_tables, context_lens, out, workspace, k_cache, v_cache,
                 scale: float, max_context_len: int, batch_sizes, split_waves: int = 0, stream=None):
        import ctypes

        if workspace is None:
            raise TypeError("workspace is required")
        if out is None:
            raise TypeError("out is required")
        _want(q, "q", _BF16, 3)
        sizes_list = [int(b) for b in batch_sizes]
        if not sizes_list or min(sizes_list) < 1:
            raise ValueError(f"batch_sizes must be positive, got {sizes_list}")
        rows = int(q.shape[0])
        if max(sizes_list) > rows:
            raise ValueError(f"the step buffers hold {rows} rows, fewer than the largest batch size {max(sizes_list)}")
        dev = _decode_args(q, k_cache, v_cache, block_tables, context_lens, out, workspace, k_new, v_new, True)
        lib = _lib.load()
        self._lib = lib
        nb, bs, hkv, d = k_cache.shape
        self.live_batch = torch.zeros(1, dtype=torch.int32, device=dev)
        self._keep = (q, k_new, v_new, block_tables, context_lens, out, workspace, k_cache, v_cache)
        st = _lib.DecodeStep(
            q=_ptr(q), q_seq_stride=_rows(q, "q"), k_new=_ptr(k_new), k_token_stride=_rows(k_new, "k_new"),
            v_new=_ptr(v_new), v_token_stride=_rows(v_new, "v_new"), live_batch=_ptr(self.live_batch),
            block_tables=_ptr(block_tables), max_blocks_per_seq=int(block_tables.shape[1]),
            context_lens=_ptr(context_lens), out=_ptr(out), workspace=_ptr(workspace),
            workspace_bytes=workspace.numel() * workspace.element_size(), k_cache=_ptr(k_cache),
            v_cache=_ptr(v_cache), block_size=bs, num_q_heads=int(q.shape[1]), num_kv_heads=hkv, head_dim=d,
            scale=float(scale), max_context_len=int(max_context_len), split_waves=int(split_waves))
        sizes = (ctypes.c_int32 * len(sizes_list))(*sizes_list)
        h = ctypes.c_void_p()
        _check("pa_decode_graphs_create", lib.pa_decode_graphs_create(
            ctypes.byref(st), sizes, len(sizes_list), _stream(stream, dev), ctypes.byref(h)))
        self._h = h
        self.batch_sizes = sizes_list
        self.device = dev

    def launch(self, batch: int, stream=None, live_written: bool = False) -> int:
        """One decode step of `batch` sequences; returns the padded batch size replayed.

        Unless live_written, batch is first written to live_batch on the launch stream (one small
        fill); a caller that writes it with the step's other inputs passes live_written=True, and
        the step is then a single graph launch.
        """
        import ctypes

        s = _stream(stream, self.device)
        if not live_written:
            with torch.cuda.stream(torch.cuda.ExternalStream(s, device=self.device)):
                self.live_batch.fill_(int(batch))
        padded = ctypes.c_int32(0)
        _check("pa_decode_graphs_launch", self._lib.pa_decode_graphs_launch(self._h, int(batch), s,
                                                                            ctypes.byref(padded)))
        return padded.value

    def close(self) -> None:
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._lib.pa_decode_graphs_destroy(h)
        self._h = None

    def __del__(self):
        self.close()
