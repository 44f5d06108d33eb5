"""The Python binding rejects arguments the C ABI cannot check (it only sees pointers): wrong
dtype, rank, contiguity or device. These run without a GPU: the checks come before any launch."""

import pytest
import torch

import paged_kv_cache_heads_amd as pa


def _cpu(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_want_rejects_wrong_dtype_rank_contiguity_and_device():
    w = pa._want
    with pytest.raises(TypeError):
        w(None, "x", torch.int32)
    assert w(None, "x", torch.int32, optional=True) is None
    with pytest.raises(TypeError):
        w([1, 2], "x", torch.int32)
    with pytest.raises(TypeError):
        w(_cpu((4,), torch.int64), "x", torch.int32)
    with pytest.raises(ValueError):
        w(_cpu((4, 2), torch.int32), "x", torch.int32, dim=1)
    with pytest.raises(ValueError):
        w(_cpu((4, 4), torch.int32).t(), "x", torch.int32, dim=2, contiguous=True)
    with pytest.raises(ValueError, match="GPU"):
        w(_cpu((4,), torch.int32), "x", torch.int32, dim=1, contiguous=True)


def test_entry_points_check_before_launching():
    bf, i32 = torch.bfloat16, torch.int32
    q, cache = _cpu((2, 16, 128), bf), _cpu((4, 256, 8, 128), bf)
    tables, lens = _cpu((2, 1), i32), _cpu((2,), i32)
    # (without a GPU every tensor is a host tensor, so only the first argument checked can show a
    # dtype error; the device check of that argument fires before later arguments are looked at)
    with pytest.raises(TypeError):  # fp16 queries
        pa.pa_decode(q.half(), cache, cache, tables, lens, 0.1, 256)
    with pytest.raises(ValueError, match="GPU"):  # host tensors
        pa.pa_decode(q, cache, cache, tables, lens, 0.1, 256)
    with pytest.raises(ValueError, match="GPU"):
        pa.pa_store_decode(q, _cpu((2, 8, 128), bf), _cpu((2, 8, 128), bf), cache, cache, tables, lens, 0.1, 256)
    with pytest.raises(TypeError):  # fp32 cache
        pa.pa_store_kvcache(_cpu((2, 8, 128), bf), _cpu((2, 8, 128), bf), cache.float(), cache, lens)
    with pytest.raises(ValueError):
        pa.pa_prefill_varlen(q, _cpu((2, 8, 128), bf), _cpu((2, 8, 128), bf), _cpu((2,), i32), _cpu((2,), i32),
                             2, 2, 0.1)
    with pytest.raises(TypeError):
        pa.pa_sample_gumbel(_cpu((2, 100), bf), _cpu((2,), torch.float32), 1, 0)
