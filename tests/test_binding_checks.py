"""The Python binding rejects arguments the C ABI cannot check (it only sees pointers): wrong
dtype, rank, contiguity, shapes that disagree across arguments, or a tensor off the GPU. These
run without a GPU: every check comes before any launch, and the shape checks come before the
device check, so host tensors of mismatched shapes are reported as shape errors."""

import pytest
import torch

import paged_kv_cache_heads_amd as pa

BF, I32, F32, U8 = torch.bfloat16, torch.int32, torch.float32, torch.uint8


def _cpu(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_want_rejects_wrong_dtype_rank_and_contiguity():
    w = pa._want
    with pytest.raises(TypeError):
        w(None, "x", I32)
    assert w(None, "x", I32, optional=True) is None
    with pytest.raises(TypeError):
        w([1, 2], "x", I32)
    with pytest.raises(TypeError):
        w(_cpu((4,), torch.int64), "x", I32)
    with pytest.raises(ValueError):
        w(_cpu((4, 2), I32), "x", I32, dim=1)
    with pytest.raises(ValueError):
        w(_cpu((4, 4), I32).t(), "x", I32, dim=2, contiguous=True)


def test_device_check_rejects_host_tensors():
    with pytest.raises(ValueError, match="GPU"):
        pa._device(x=_cpu((4,), I32))
    assert pa._device(x=None) is None


def test_shape_helper():
    pa._shape(_cpu((3, 4), I32), "x", (3, None))
    pa._shape(None, "x", (1,))
    with pytest.raises(ValueError, match=r"\(3, 5\)"):
        pa._shape(_cpu((3, 4), I32), "x", (3, 5))
    with pytest.raises(ValueError):
        pa._shape(_cpu((3, 4), I32), "x", (3, 4, 1))


# ---- well-formed host arguments: only the device check fails


def _decode_ok(b=2):
    return dict(q=_cpu((b, 16, 128), BF), k_cache=_cpu((4, 256, 8, 128), BF), v_cache=_cpu((4, 256, 8, 128), BF),
                block_tables=_cpu((b, 1), I32), context_lens=_cpu((b,), I32))


def test_well_formed_arguments_reach_the_device_check():
    a = _decode_ok()
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_decode(a["q"], a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1, 256)
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_store_decode(a["q"], _cpu((2, 8, 128), BF), _cpu((2, 8, 128), BF), a["k_cache"], a["v_cache"],
                           a["block_tables"], a["context_lens"], 0.1, 256)
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_store_kvcache(_cpu((3, 8, 128), BF), _cpu((3, 8, 128), BF), a["k_cache"], a["v_cache"],
                            _cpu((3,), I32))
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_prefill_varlen(_cpu((5, 16, 128), BF), _cpu((5, 8, 128), BF), _cpu((5, 8, 128), BF),
                             _cpu((2,), I32), _cpu((2,), I32), 5, 5, 0.1)
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_sample_gumbel(_cpu((2, 100), F32), _cpu((2,), F32), 1, 0)
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_qk_norm_rope_store(_cpu((3, 32 * 128), BF), _cpu((128,), BF), _cpu((128,), BF), 1e-6,
                                 _cpu((64, 128), F32), _cpu((3,), I32), a["k_cache"], a["v_cache"], _cpu((3,), I32),
                                 16)


def test_dtype_errors_come_first():
    a = _decode_ok()
    with pytest.raises(TypeError):  # fp16 queries
        pa.pa_decode(a["q"].half(), a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1, 256)
    with pytest.raises(TypeError):  # fp32 cache
        pa.pa_store_kvcache(_cpu((2, 8, 128), BF), _cpu((2, 8, 128), BF), a["k_cache"].float(), a["v_cache"],
                            _cpu((2,), I32))
    with pytest.raises(TypeError):
        pa.pa_sample_gumbel(_cpu((2, 100), BF), _cpu((2,), F32), 1, 0)


# ---- one mismatched shape per case: a ValueError naming the argument, before the device check


@pytest.mark.parametrize("name,bad", [
    ("block_tables", _cpu((1, 1), I32)),      # fewer rows than sequences
    ("context_lens", _cpu((1,), I32)),
    ("v_cache", _cpu((4, 256, 4, 128), BF)),  # other head count than k_cache
    ("k_cache", _cpu((4, 256, 8, 64), BF)),   # other head_dim than q (v_cache alike)
])
def test_decode_shape_mismatch(name, bad):
    a = _decode_ok()
    a[name] = bad
    if name == "k_cache":
        a["v_cache"] = bad
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        pa.pa_decode(a["q"], a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1, 256)


def test_decode_out_shape_mismatch():
    a = _decode_ok()
    with pytest.raises(ValueError, match="out must have shape"):
        pa.pa_decode(a["q"], a["k_cache"], a["v_cache"], a["block_tables"], a["context_lens"], 0.1, 256,
                     out=_cpu((1, 16, 128), BF))


@pytest.mark.parametrize("which", ["k_new", "v_new"])
def test_store_decode_new_rows_mismatch(which):
    a = _decode_ok()
    kv = {"k_new": _cpu((2, 8, 128), BF), "v_new": _cpu((2, 8, 128), BF)}
    kv[which] = _cpu((1, 8, 128), BF)
    with pytest.raises(ValueError, match=f"{which} must have shape"):
        pa.pa_store_decode(a["q"], kv["k_new"], kv["v_new"], a["k_cache"], a["v_cache"], a["block_tables"],
                           a["context_lens"], 0.1, 256)


@pytest.mark.parametrize("case", ["k_rows", "v_heads", "v_cache", "slots"])
def test_store_shape_mismatch(case):
    k, v = _cpu((3, 8, 128), BF), _cpu((3, 8, 128), BF)
    kc, vc, slots = _cpu((4, 256, 8, 128), BF), _cpu((4, 256, 8, 128), BF), _cpu((3,), I32)
    if case == "k_rows":
        k = _cpu((2, 8, 128), BF)
    elif case == "v_heads":
        v = _cpu((3, 4, 128), BF)
    elif case == "v_cache":
        vc = _cpu((2, 256, 8, 128), BF)
    else:
        slots = _cpu((5,), I32)
    with pytest.raises(ValueError, match="shape"):
        pa.pa_store_kvcache(k, v, kc, vc, slots)


@pytest.mark.parametrize("case", ["cu_k", "out", "k_dim", "v_shape", "table_rows"])
def test_prefill_shape_mismatch(case):
    q, k, v = _cpu((5, 16, 128), BF), _cpu((5, 8, 128), BF), _cpu((5, 8, 128), BF)
    cu_q, cu_k, out, table = _cpu((2,), I32), _cpu((2,), I32), None, None
    if case == "cu_k":
        cu_k = _cpu((3,), I32)
    elif case == "out":
        out = _cpu((4, 16, 128), BF)
    elif case == "k_dim":
        k = v = _cpu((5, 8, 64), BF)
    elif case == "v_shape":
        v = _cpu((6, 8, 128), BF)
    else:
        k = v = _cpu((4, 256, 8, 128), BF)
        table = _cpu((3, 1), I32)
    with pytest.raises(ValueError, match="shape"):
        pa.pa_prefill_varlen(q, k, v, cu_q, cu_k, 5, 5, 0.1, block_table=table, out=out)


@pytest.mark.parametrize("case", ["qkv_width", "cos_sin", "positions", "slots", "weight", "q_out", "v_cache"])
def test_norm_rope_shape_mismatch(case):
    args = dict(qkv=_cpu((3, 32 * 128), BF), qw=_cpu((128,), BF), kw=_cpu((128,), BF), cs=_cpu((64, 128), F32),
                pos=_cpu((3,), I32), kc=_cpu((4, 256, 8, 128), BF), vc=_cpu((4, 256, 8, 128), BF),
                slots=_cpu((3,), I32), q_out=None)
    bad = {"qkv_width": ("qkv", _cpu((3, 30 * 128), BF)), "cos_sin": ("cs", _cpu((64, 64), F32)),
           "positions": ("pos", _cpu((2,), I32)), "slots": ("slots", _cpu((4,), I32)),
           "weight": ("kw", _cpu((64,), BF)), "q_out": ("q_out", _cpu((3, 8, 128), BF)),
           "v_cache": ("vc", _cpu((4, 256, 4, 128), BF))}[case]
    args[bad[0]] = bad[1]
    with pytest.raises(ValueError, match="shape"):
        pa.pa_qk_norm_rope_store(args["qkv"], args["qw"], args["kw"], 1e-6, args["cs"], args["pos"], args["kc"],
                                 args["vc"], args["slots"], 16, q_out=args["q_out"])


@pytest.mark.parametrize("case", ["temps", "tokens"])
def test_sampler_shape_mismatch(case):
    temps = _cpu((1,), F32) if case == "temps" else _cpu((2,), F32)
    tokens = _cpu((3,), I32) if case == "tokens" else None
    with pytest.raises(ValueError, match="shape"):
        pa.pa_sample_gumbel(_cpu((2, 100), F32), temps, 1, 0, tokens=tokens)


def test_decode_graphs_buffers_must_hold_the_largest_batch():
    a = _decode_ok(4)
    kv = _cpu((4, 8, 128), BF)
    common = (a["q"], kv, kv, a["block_tables"], a["context_lens"], _cpu((4, 16, 128), BF), _cpu((1024,), U8),
              a["k_cache"], a["v_cache"], 0.1, 256)
    with pytest.raises(ValueError, match="largest batch"):
        pa.DecodeGraphs(*common, [2, 8])
    bad = list(common)
    bad[4] = _cpu((3,), I32)  # context_lens shorter than the step buffers
    with pytest.raises(ValueError, match="context_lens"):
        pa.DecodeGraphs(*bad, [2, 4])
