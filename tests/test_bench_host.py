"""Host-side logic of bench.py: the work counts its rates divide by, the one-GPU guard and the oracle baseline."""

import json
import os
import subprocess
import sys

import torch

import bench
from workloads import configs, tensors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    msg = json.loads(res.stdout.strip().splitlines()[-1])
    assert "error" in msg and msg["n_gpus"] == 2


def test_decode_bytes_tiny_workload():
    # context lengths 1, 37, 256, 300: 594 tokens, each a K and a V row of 8 heads x 128 bf16 values
    wl = configs.config1()
    b = bench.decode_bytes(wl)
    assert b["kv"] == 594 * 8 * 128 * 2 * 2
    q_out = 4 * 16 * 128 * 2 * 2
    tables = (1 + 1 + 1 + 2) * 4  # ceil(L / 256) entries per sequence
    assert b["total"] == b["kv"] + q_out + tables + 4 * 4


def test_store_bytes():
    wl = configs.config1()
    # per token: K and V rows read and written (2 x 2 x 2048 bytes) and the 4-byte slot
    assert bench.store_bytes(wl, 10) == 10 * (4 * 2048 + 4)


def test_prefill_flops_counts_unmasked_pairs():
    hq, d = 4, 128
    wl = configs.prefill_workload("f", [1, 5], 0, hq, 2, 16, seed=1)
    # causal, queries aligned with keys: n (n + 1) / 2 visible pairs per sequence
    assert bench.prefill_flops(wl) == (1 + 15) * 4 * d * hq
    assert bench.prefill_flops(wl, causal=False) == (1 + 25) * 4 * d * hq
    wl = configs.prefill_workload("p", [3], 64, hq, 2, 16, seed=1, block_size=64)
    # 3 queries after a 64-token prefix: each sees the prefix and the queries up to itself
    assert bench.prefill_flops(wl) == (64 * 3 + 6) * 4 * d * hq
    assert bench.prefill_flops(wl, causal=False) == 3 * 67 * 4 * d * hq


def test_norm_rope_bytes():
    wl = configs.config1()
    heads = 16 + 2 * 8
    per_token = heads * 128 * 2 * 2 + 128 * 4 + 8
    assert bench.norm_rope_bytes(wl, 3) == 3 * per_token + 2 * 128 * 2


def test_balanced_shares():
    shares = bench.balanced_shares([5, 1, 1, 1, 1, 1, 4], 3)
    assert sorted(i for g in shares for i in g) == list(range(7))
    loads = sorted(sum([5, 1, 1, 1, 1, 1, 4][i] for i in g) for g in shares)
    assert loads == [4, 5, 5]
    assert bench.balanced_shares([3], 4) == [[0]]


def test_oracle_baselines_on_a_worker_pool():
    # the unmodified oracle over shares of each batch, in spawned worker processes
    pool = bench.start_oracle_pool(2)
    try:
        cpu = torch.device("cpu")
        wl = configs.prefill_workload("cpu", [20, 7, 13], 0, 16, 8, 16, seed=2)
        r = bench.run_oracle_baseline(pool, *bench.prefill_tasks(tensors.materialize(wl, cpu), wl, 2, paged=False),
                                      "TFLOP/s", "packed")
        assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["cores"] == 2 and r["value"] > 0
        assert r["oracle_s_slowest_share"] <= r["oracle_s_all_shares"]
        wl = configs.prefill_workload("cpu-prefix", [9, 30], 64, 16, 8, 16, seed=3, block_size=64)
        tasks, work = bench.prefill_tasks(tensors.materialize(wl, cpu), wl, 2, paged=True)
        assert sum(work) == bench.prefill_flops(wl)
        assert bench.run_oracle_baseline(pool, tasks, work, "TFLOP/s", "paged")["value"] > 0
        wl = configs.decode_workload("cpu-decode", [5, 300, 40, 1], 16, 8, 8, seed=4)
        tasks, work = bench.decode_tasks(tensors.materialize(wl, cpu), wl, [0, 1, 3], 2)
        assert sum(work) == (5 + 300 + 1) * 8 * 128 * 4
        r = bench.run_oracle_baseline(pool, tasks, work, "GB/s", "decode")
        assert r["unit"] == "GB/s" and r["cores"] == 2 and r["value"] > 0
    finally:
        pool.terminate()
        pool.join()


def test_traffic_gate_hashes_every_decode_source():
    """The recorded decode traffic is reported only while the decode kernels' sources hash to the
    recorded value; every local header decode.hip pulls in (recursively) must be part of that hash."""
    import re
    csrc = os.path.join(ROOT, "paged_kv_cache_heads_amd", "csrc")
    seen, todo = set(), ["decode.hip"]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        for inc in re.findall(r'^#include "([^"]+)"', open(os.path.join(csrc, name)).read(), re.M):
            if not inc.startswith("../"):
                todo.append(inc)
    assert {"csrc/" + n for n in seen} <= set(bench.DECODE_SOURCES), seen
    assert "build.py" in bench.DECODE_SOURCES
    assert len(bench.decode_source_sha()) == 16
