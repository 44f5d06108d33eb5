"""One tensor-parallel shard's shape on one GPU: with the kv heads split over 8 GPUs, each GPU runs the same
kernels at one kv head (Hq 2 / Hkv 1 for the Qwen3-0.6B layout, Hq 4 / Hkv 1 for the long-context layout).
Store, decode and prefill at those shapes against the oracle."""

import numpy as np
import pytest

from tests.gpu_common import announce, dev  # noqa: F401
from tests.test_gpu_decode import _run
from tests.test_gpu_prefill import _packed, _table
from workloads import configs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("split_waves", [0, 300])
def test_decode_shard_qwen_layout(dev, split_waves):
    announce(f"decode TP shard Hq 2 / Hkv 1, waves {split_waves}")
    lens = np.random.default_rng(31).integers(100, 2049, 64)
    nb = int(sum(-(-int(n) // 256) for n in lens)) + 8
    wl = configs.decode_workload("tp-decode", lens, 2, 1, nb, seed=31)
    _run(wl, dev, split_waves=split_waves)


def test_decode_shard_long_context_layout(dev):
    announce("decode TP shard Hq 4 / Hkv 1, long contexts")
    rng = np.random.default_rng(33)
    lens = np.clip(np.floor(np.exp(rng.uniform(np.log(256), np.log(16384), 24))), 256, 16384).astype(int)
    nb = int(sum(-(-int(n) // 256) for n in lens)) + 8
    wl = configs.decode_workload("tp-long", lens, 4, 1, nb, seed=33)
    _run(wl, dev)


@pytest.mark.parametrize("max_k", [None, 4096])
def test_prefill_shard_varlen(dev, max_k):
    announce(f"prefill TP shard Hq 2 / Hkv 1, max_k {max_k}")
    lens = [int(x) for x in np.random.default_rng(32).integers(100, 1025, 12)]
    nb = sum(-(-n // 256) for n in lens) + 4
    wl = configs.prefill_workload("tp-prefill", lens, 0, 2, 1, nb, seed=32)
    _packed(wl, dev, max_k=max_k)


def test_prefill_shard_prefix(dev):
    announce("prefix-cached prefill TP shard Hq 2 / Hkv 1")
    lens = [int(x) for x in np.random.default_rng(34).integers(128, 513, 8)]
    nb = 4 + sum(-(-(1024 + n) // 256) - 4 for n in lens) + 4
    wl = configs.prefill_workload("tp-prefix", lens, 1024, 2, 1, nb, seed=34)
    _table(wl, dev)
