"""Benchmark of the paged-KV-cache attention path on one MI355X.

One step is one pass of the whole path over seeded synthetic batches:
  decode leg       store 256 new tokens + paged decode (256 seqs, L ~ U{100..2048},
                   Hq 16 / Hkv 8 / D 128, 256-token blocks, 4096-block pool), one
                   pa_store_decode call (the separate pa_store_kvcache + pa_decode
                   calls are timed after the steps and reported beside);
  long decode leg  the same step for the long-context batch: 512 seqs, Hq 32 / Hkv 8
                   (G = 4), L log-uniform in [256, 32768], a 164,794-block pool
                   (60% of HBM for one layer's K and V); the split-K decode;
  prefill leg      store + causal varlen prefill over packed q/k/v (about 29 seqs
                   of 100..1024 tokens, at most 16384 tokens);
  prefix leg       store + prefix-cached prefill through the block table (32 seqs
                   sharing 1024 cached tokens, 128..512 new tokens each);
  fused leg        QK-RMSNorm + rotary embedding + store of the prefill batch's
                   q/k/v (one pass, reported as its own roofline);
  sampler leg      Gumbel-max sampling of one token for each of the 256 decode
                   sequences over a 151936-token vocabulary (fp32 logits).
After the timed steps (outside them): the decode legs as two separate calls,
the prefill legs as one fused store + prefill call against the separate pair,
the varlen batch's store beside torch's index_copy_ scatter and a contiguous
copy of the same bytes,
host timings of the C++ block manager, the wall-clock decode-step latency eager
vs graph-captured at batch 1, 16 and 256, and the fp64 oracle timed on the
host's cores over the decode, prefill, prefix and long-decode batches.
Inputs are resident in HBM before timing starts. `value` is the decode leg's
KV-read throughput (bytes of K and V the decode must read, over the leg's
time); the prefill legs report TFLOP/s of unmasked query-key pairs. Kernel
times come from HIP events recorded on the launch stream around each call.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn KV-read GB/s (% HBM peak); prefill attn TFLOP/s (% MFMA)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
SAMPLER_VOCAB = 151936          # vocabulary of the Qwen3 family the pages benchmark
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
# The pages' end-to-end figure, quoted as context (other hardware, whole engine, not this path's metric):
# nano-vLLM offline generation of Qwen3-0.6B over 256 random-length requests on a laptop RTX 4070
# (page "nano-vLLM 最小化vLLM重新实现", 基准测试).
PAGES_END_TO_END = {"value": 1434, "unit": "tok/s", "model": "Qwen3-0.6B", "sequences": 256,
                    "hardware": "RTX 4070 laptop GPU", "what": "whole-engine offline generation, 133,966 tokens "
                    "in 93.41 s; context only, not comparable with this path's kernel metric"}


# ----------------------------------------------------------------------------- timing events
#
# Kernel times come from HIP events recorded on the launch stream. torch's events carry a system-scope
# fence (an L2 writeback and invalidate) that costs about 1.5 us of GPU time per event span, 6% of a
# 25 us store launch; the HIP runtime documents hipEventDisableSystemFence for such timing. These events
# are created through the HIP runtime that torch itself has loaded (found in the process map, so that the
# events and torch's streams belong to one runtime) and are used only for timestamps.

_HIP = None
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def _hip_runtime():
    global _HIP
    if _HIP is None:
        import ctypes
        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if ln.rstrip().endswith("libamdhip64.so")
                     or "libamdhip64.so." in ln), None)
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        lib = ctypes.CDLL(path)
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = lib
    return _HIP


class TimingEvent:
    """A HIP timing event without the system-scope fence, with torch.cuda.Event's record() /
    elapsed_time() interface (milliseconds), recorded on torch's current stream."""

    def __init__(self):
        import ctypes
        self._ctypes = ctypes
        self._hip = _hip_runtime()
        self._e = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self._e), _HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        rc = self._hip.hipEventRecord(self._e, self._ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        ms = self._ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(self._ctypes.byref(ms), self._e, end._e)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if getattr(self, "_e", None) is not None and self._e.value:
            self._hip.hipEventDestroy(self._e)
            self._e = None


def decode_bytes(wl) -> dict:
    """Algorithmic bytes of one decode launch: every context token's K and V row
    of the kv heads, plus q in, out, the used table entries and the lengths."""
    row = wl.num_kv_heads * wl.head_dim * 2
    kv = int(wl.context_lens.astype(np.int64).sum()) * row * 2
    qo = wl.num_seqs * wl.num_q_heads * wl.head_dim * 2 * 2
    tables = sum(-(-int(n) // wl.block_size) for n in wl.context_lens) * 4
    return {"kv": kv, "total": kv + qo + tables + wl.num_seqs * 4}


def store_bytes(wl, n_tokens) -> int:
    row = wl.num_kv_heads * wl.head_dim * 2
    return n_tokens * (2 * row * 2 + 4)


def norm_rope_bytes(wl, n_tokens) -> int:
    """Algorithmic bytes of one fused QK-norm + rotary + store launch: the qkv row in,
    q out, K and V rows to the cache, the position's cos/sin row, position and slot."""
    d = wl.head_dim
    heads = wl.num_q_heads + 2 * wl.num_kv_heads
    per_token = heads * d * 2 * 2 + d * 4 + 4 + 4
    return n_tokens * per_token + 2 * d * 2


def prefill_flops(wl, causal=True) -> int:
    """4 * D * Hq flops per unmasked (query, key) pair (q.k and p.v)."""
    nq = np.diff(wl.cu_seqlens_q).astype(np.int64)
    nk = np.diff(wl.cu_seqlens_k).astype(np.int64)
    pairs = 0
    for a, b in zip(nq, nk):
        pairs += int((b - a) * a + a * (a + 1) // 2) if causal else int(a * b)
    return pairs * 4 * wl.head_dim * wl.num_q_heads


def separate_decode_leg(pa, torch, b, wl, scale, max_len, ws, out, steps, warmup, split_waves=0):
    """A decode leg as pa_store_kvcache + pa_decode (two launches), median over the step count."""
    def once(ev=None):
        if ev is not None:
            ev[0].record()
        pa.pa_store_kvcache(b.k_new, b.v_new, b.k_cache, b.v_cache, b.slot_mapping)
        if ev is not None:
            ev[1].record()
        pa.pa_decode(b.q, b.k_cache, b.v_cache, b.block_tables, b.context_lens, scale, max_len, out=out,
                     workspace=ws, split_waves=split_waves)
        if ev is not None:
            ev[2].record()
    for _ in range(warmup):
        once()
    torch.cuda.synchronize()
    evs = [[TimingEvent() for _ in range(3)] for _ in range(steps)]
    for e in evs:
        once(e)
    torch.cuda.synchronize()
    st = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    dt = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    kv = decode_bytes(wl)["kv"]
    return {"store_us": round(st * 1e3, 2), "decode_us": round(dt * 1e3, 2),
            "kv_GBs_leg": round(kv / ((st + dt) * 1e-3) / 1e9, 1),
            "decode_GBs": round(decode_bytes(wl)["total"] / (dt * 1e-3) / 1e9, 1)}


def back_to_back_us(torch, fn, reps=10, rounds=7, warmup=2):
    """Median over `rounds` of the mean time per call of `reps` back-to-back calls between two events on
    the current stream: the GPU stays busy, so host launch costs between calls are hidden as in a step."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    per = []
    for _ in range(rounds):
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / reps)
    return float(np.median(per))


def fused_store_prefill(pa, torch, scale, b3, wl3, b4, wl4, out3, out4):
    """The two prefill legs as one pa_store_prefill_varlen call against pa_store_kvcache + pa_prefill_varlen
    (time per call of back-to-back calls, the two forms alternating)."""
    legs = {
        "varlen": (lambda: (pa.pa_store_kvcache(b3.k_new, b3.v_new, b3.k_cache, b3.v_cache, b3.slot_mapping),
                            pa.pa_prefill_varlen(b3.q, b3.k_new, b3.v_new, b3.cu_seqlens_q, b3.cu_seqlens_k,
                                                 wl3.max_seqlen_q, wl3.max_seqlen_k, scale, out=out3)),
                   lambda: pa.pa_store_prefill_varlen(b3.q, b3.k_new, b3.v_new, b3.k_cache, b3.v_cache,
                                                      b3.slot_mapping, b3.cu_seqlens_q, b3.cu_seqlens_k,
                                                      wl3.max_seqlen_q, wl3.max_seqlen_k, scale, out=out3)),
        "prefix": (lambda: (pa.pa_store_kvcache(b4.k_new, b4.v_new, b4.k_cache, b4.v_cache, b4.slot_mapping),
                            pa.pa_prefill_varlen(b4.q, b4.k_cache, b4.v_cache, b4.cu_seqlens_q, b4.cu_seqlens_k,
                                                 wl4.max_seqlen_q, wl4.max_seqlen_k, scale,
                                                 block_table=b4.block_tables, out=out4)),
                   lambda: pa.pa_store_prefill_varlen(b4.q, b4.k_new, b4.v_new, b4.k_cache, b4.v_cache,
                                                      b4.slot_mapping, b4.cu_seqlens_q, b4.cu_seqlens_k,
                                                      wl4.max_seqlen_q, wl4.max_seqlen_k, scale,
                                                      block_table=b4.block_tables, out=out4)),
    }
    res = {}
    for name, (unfused, fused) in legs.items():
        t = {"unfused": [], "fused": []}
        for i in range(3):  # alternate the two forms
            t["unfused"].append(back_to_back_us(torch, unfused))
            t["fused"].append(back_to_back_us(torch, fused))
        res[name] = {"store_then_prefill_us": round(float(np.median(t["unfused"])), 2),
                     "fused_us": round(float(np.median(t["fused"])), 2)}
    return res


def store_references(pa, torch, b3, wl3):
    """The varlen batch's store (15.8k tokens, 130 MB moved) beside references over the same bytes: the
    same scatter done by torch (index_copy_ of the K rows and of the V rows into the caches by slot), a
    plain contiguous device copy of the same byte count (no indirection, no stride), and torch copying the
    store's own source rows (K and V of each token, 4 KiB at the fused projection's 8 KiB row stride) into
    contiguous memory: the same reads, contiguous writes. Time per call of back-to-back calls, the four
    alternating."""
    hkv, d = wl3.num_kv_heads, wl3.head_dim
    slots = b3.slot_mapping.long()
    kflat, vflat = b3.k_cache.view(-1, hkv, d), b3.v_cache.view(-1, hkv, d)
    src = torch.empty((wl3.num_tokens, 2 * hkv * d), dtype=torch.bfloat16, device=b3.q.device)
    dst = torch.empty_like(src)
    # the store's own source rows: each token's K and V, 4 KiB of every fused-projection row
    kv_rows = b3.qkv[:, wl3.num_q_heads * d:]
    calls = {
        "pa_store_kvcache": lambda: pa.pa_store_kvcache(b3.k_new, b3.v_new, b3.k_cache, b3.v_cache, b3.slot_mapping),
        "torch_index_copy": lambda: (kflat.index_copy_(0, slots, b3.k_new), vflat.index_copy_(0, slots, b3.v_new)),
        "contiguous_copy": lambda: dst.copy_(src),
        "strided_source_copy": lambda: dst.copy_(kv_rows),
    }
    t = {k: [] for k in calls}
    for i in range(3):  # alternate the three
        for k, fn in calls.items():
            t[k].append(back_to_back_us(torch, fn))
    nbytes = store_bytes(wl3, wl3.num_tokens)
    res = {k: {"us": round(float(np.median(v)), 2), "GBs": round(nbytes / (float(np.median(v)) * 1e-6) / 1e9, 1)}
           for k, v in t.items()}
    res["bytes"] = nbytes
    res["speedup_vs_torch"] = round(res["torch_index_copy"]["us"] / res["pa_store_kvcache"]["us"], 2)
    del src, dst
    return res


def measured_peaks(torch, dev):
    """Ceilings measured on this GPU after the timed steps (best of 10): a 1 GiB device-to-device copy
    (read + written bytes) and a bf16 8192^3 matrix product through torch.matmul (the vendor GEMM),
    reported beside the spec peaks. The prefill rooflines also give their fraction of the GEMM rate. The
    copy is context only: it mixes reads and writes and runs below the decode kernel's pure read stream."""
    def best_ms(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            a, b = TimingEvent(), TimingEvent()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        return best
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_gbs = 2 * src.numel() / (best_ms(lambda: dst.copy_(src)) * 1e-3) / 1e9
    del src, dst
    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    y = torch.randn((n, n), dtype=torch.bfloat16, device=dev).contiguous()
    gemm_tflops = 2 * n ** 3 / (best_ms(lambda: torch.matmul(x, y)) * 1e-3) / 1e12
    del x, y
    return {"copy_GBs": round(copy_gbs, 1), "bf16_gemm_TFLOPs": round(gemm_tflops, 1),
            "note": "1 GiB device copy (read + write bytes); torch.matmul bf16 8192^3; best of 10"}


# The decode kernels' source and every local header it includes (csrc/), then the build flags.
DECODE_SOURCES = ("csrc/decode.hip", "csrc/common.h", "csrc/launch.h", "csrc/mfma_tiles.h", "build.py")


def decode_source_sha() -> str:
    """Hash of the decode kernels' sources and build flags: a recorded counter figure is only
    reported while it still describes the code being run."""
    import hashlib
    srcs = [os.path.join(ROOT, "paged_kv_cache_heads_amd", n) for n in DECODE_SOURCES]
    return hashlib.sha256(b"".join(open(p, "rb").read() for p in srcs)).hexdigest()[:16]


def measured_traffic(leg: str):
    """HBM bytes per launch of a decode leg ("decode" or "long_decode") from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, or None if the decode kernel sources or the compile flags changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "bench_default_hbm_traffic.md")
    try:
        recs = []
        with open(path, encoding="utf-8") as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    recs.append(json.loads(line.split(":", 1)[1]))
        sha = decode_source_sha()
    except OSError:
        return None
    for rec in recs:
        if rec.get("leg") == leg and rec.get("source_sha256_16") == sha:
            return rec["bytes_per_launch"]
    return None


def host_block_manager(wl2, wl4, reps=20):
    """Host timings of the C++ block manager on the bench's batches (best of reps):
    allocating the prefix batch's 32 prompts (1024 shared tokens reused from the
    cache after the first), one decode step for the 256-sequence batch (one batched
    append plus its decode metadata), and XXH64 throughput over 1 MiB."""
    from paged_kv_cache_heads_amd.blocks import BlockManager, xxh64

    rng = np.random.default_rng(5)
    prefix = rng.integers(0, 32000, 1024).tolist()
    prompts = [np.asarray(prefix + rng.integers(0, 32000, int(n) - 1024).tolist(), dtype=np.int32)
               for n in np.diff(wl4.cu_seqlens_k)]
    alloc, cached = [], 0
    for _ in range(reps):
        bm = BlockManager(wl4.num_blocks, wl4.block_size)
        t0 = time.perf_counter()
        cached = sum(bm.allocate(i, p) for i, p in enumerate(prompts))
        alloc.append(time.perf_counter() - t0)
    bm = BlockManager(wl2.num_blocks, wl2.block_size)
    for i, n in enumerate(wl2.context_lens):
        bm.allocate(i, rng.integers(0, 32000, max(int(n) - 1, 0)).tolist())
    ids = np.arange(wl2.num_seqs, dtype=np.int64)
    width = int(wl2.block_tables.shape[1])
    step = []
    for r in range(reps):
        toks = np.full(wl2.num_seqs, r, dtype=np.int32)
        t0 = time.perf_counter()
        bm.append_batch(ids, toks)
        bm.decode_metadata(ids, width + 1)
        step.append(time.perf_counter() - t0)
    data = rng.integers(0, 256, 1 << 20, dtype=np.uint8).tobytes()
    hs = []
    for _ in range(reps):
        t0 = time.perf_counter()
        xxh64(data, 0)
        hs.append(time.perf_counter() - t0)
    total_prompt = sum(len(p) for p in prompts)
    return {"allocate_prefix_batch_us": round(min(alloc) * 1e6, 1), "prefix_batch_prompt_tokens": total_prompt,
            "prefix_batch_cached_tokens": cached, "decode_step_256_seqs_us": round(min(step) * 1e6, 1),
            "xxh64_GBs": round((1 << 20) / min(hs) / 1e9, 2), "threads": 1,
            "note": "host C++ through the Python binding (call overhead included)"}


def decode_graph_latency(pa, torch, b2, wl2, scale, batches=(1, 16, 256), iters=200):
    """Wall-clock time per decode step, eager pa_store_decode through the binding vs one graph launch
    (inputs, including the graph's live count, written before the timed launches), for the first
    `batch` sequences of the decode batch: back to back on one stream (synchronised once per
    measurement), and isolated (each step launched and waited for)."""
    dev = b2.q.device
    sizes = [1, 2, 4, 8, 16, 32, 64, 128, 256]
    maxb = sizes[-1]
    w = int(b2.block_tables.shape[1])
    max_len = w * wl2.block_size
    q_s, k_s, v_s = b2.q.clone(), b2.k_new.contiguous(), b2.v_new.contiguous()
    bt_s, cl_s = b2.block_tables.clone(), b2.context_lens.clone()
    out_s = torch.empty_like(q_s)
    ws = torch.empty(pa.pa_decode_workspace_size(maxb, 16, 8, 128, max_len), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    res = {"batch": list(batches), "eager_step_us": [], "graph_step_us": [], "eager_isolated_step_us": [],
           "graph_isolated_step_us": [], "captured_sizes": sizes}
    with torch.cuda.stream(stream):
        graphs = pa.DecodeGraphs(q_s, k_s, v_s, bt_s, cl_s, out_s, ws, b2.k_cache, b2.v_cache, scale, max_len,
                                 sizes)
        for batch in batches:
            qs, ks, vs = q_s[:batch], k_s[:batch], v_s[:batch]
            bt, cl, o = bt_s[:batch], cl_s[:batch], out_s[:batch]

            def eager():
                pa.pa_store_decode(qs, ks, vs, b2.k_cache, b2.v_cache, bt, cl, scale, max_len, out=o, workspace=ws)

            graphs.live_batch.fill_(batch)
            for fn, key in ((eager, "eager"), (lambda: graphs.launch(batch, live_written=True), "graph")):
                for _ in range(10):
                    fn()
                stream.synchronize()
                # back to back: the GPU's time per step once launches queue ahead of it
                t0 = time.perf_counter()
                for _ in range(iters):
                    fn()
                stream.synchronize()
                res[key + "_step_us"].append(round((time.perf_counter() - t0) / iters * 1e6, 1))
                # isolated: launch, then wait for the step (the per-token latency a sampler waiting on
                # each step sees, launch cost included); median over the iterations
                lat = []
                for _ in range(iters):
                    t0 = time.perf_counter()
                    fn()
                    stream.synchronize()
                    lat.append(time.perf_counter() - t0)
                res[key + "_isolated_step_us"].append(round(float(np.median(lat)) * 1e6, 1))
        graphs.close()
    stream.synchronize()
    return res


LEAD_IN_US = 200.0


def lead_in_cycles(torch) -> int:
    """Argument of torch.cuda._sleep (a one-thread spin on the GPU's cycle counter) for about LEAD_IN_US,
    calibrated on this GPU with one timed spin."""
    cal = 1 << 20
    torch.cuda._sleep(1000)
    a, b = TimingEvent(), TimingEvent()
    a.record()
    torch.cuda._sleep(cal)
    b.record()
    torch.cuda.synchronize()
    us = max(a.elapsed_time(b) * 1e3, 1.0)
    return max(1, int(cal * LEAD_IN_US / us))


def cold_launches(torch, dev, kernels, calls, reps=20, warmup=5):
    """Event-timed duration (us) of each launch run alone after a 512 MiB write has flushed the L2 and
    MALL, so that no kernel finds its inputs left in cache by the one before it: `warmup` untimed calls,
    then `reps` timed ones. Returns the medians and, separately, median / min / max."""
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out, stats = {}, {}
    for name in kernels:
        t = []
        for r in range(reps + warmup):
            flush.fill_(r & 0xFF)
            e0, e1 = TimingEvent(), TimingEvent()
            e0.record()
            calls[name]()
            e1.record()
            torch.cuda.synchronize()
            if r >= warmup:
                t.append(e0.elapsed_time(e1) * 1e3)
        out[name] = round(float(np.median(t)), 2)
        stats[name] = {"median": out[name], "min": round(float(np.min(t)), 2), "max": round(float(np.max(t)), 2)}
    del flush
    return out, stats


# ----------------------------------------------------------------------------- oracle baseline (host)
#
# The fp64 oracle as it stands, timed on the host's cores. Its work is Python loops over positions,
# sequences and heads around small numpy calls, which threads cannot share, so the cores are used the
# way an unmodified single-threaded program can use them: one worker process per core (BLAS limited
# to one thread each), each running the oracle over its own share of the sequences. The pool is
# spawned before anything touches the GPU; each worker times only its oracle calls, and the rate is
# the shares' total work over the slowest worker's time.


def host_cores() -> int:
    return len(os.sched_getaffinity(0))


def start_oracle_pool(n: int):
    import multiprocessing as mp
    pool = mp.get_context("spawn").Pool(n)
    pool.map(_worker_ready, range(n))  # every worker has started (and imported numpy) before timing
    return pool


def _worker_ready(_):
    return os.getpid()


def _oracle_worker(task: dict) -> float:
    """One share of an oracle baseline, in a worker process: seconds spent in the oracle calls."""
    import threadpoolctl

    import oracle
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        if task["kind"] == "decode":
            kc, vc = oracle.store_kvcache(task["k_new"], task["v_new"], task["slots"], task["k"], task["v"])
            oracle.decode(task["q"], kc, vc, task["tables"], task["lens"], task["scale"])
        else:
            oracle.prefill_varlen(task["q"], task["k"], task["v"], task["cu_q"], task["cu_k"], task["scale"],
                                  causal=True, block_table=task.get("tables"))
        return time.perf_counter() - t0


def balanced_shares(costs, n: int):
    """Indices split into at most n groups of about equal total cost (heaviest first to the lightest)."""
    groups, load = [[] for _ in range(n)], [0] * n
    for i in sorted(range(len(costs)), key=lambda i: -costs[i]):
        j = min(range(n), key=load.__getitem__)
        groups[j].append(i)
        load[j] += costs[i]
    return [sorted(g) for g in groups if g]


def decode_tasks(batch, wl, seqs, n: int):
    """Store + decode of the given sequences, split in n shares, each with a host copy of its blocks."""
    from tests.parity import Compact  # test infrastructure, used only for this leg
    from workloads import tensors

    q, k_new, v_new = tensors.to_u16(batch.q), tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new)
    slots = batch.slot_mapping.cpu().numpy()
    lens = wl.context_lens.astype(np.int64)
    tasks, work = [], []
    for share in balanced_shares([int(lens[s]) for s in seqs], n):
        ss = [int(seqs[i]) for i in share]
        host = Compact(batch, ss)
        tasks.append({"kind": "decode", "q": q[ss], "k_new": k_new[ss], "v_new": v_new[ss],
                      "slots": np.array([host.remap_slot(int(slots[s]), wl.block_size) for s in ss], np.int64),
                      "k": host.k, "v": host.v, "tables": host.tables, "lens": lens[ss],
                      "scale": 1.0 / math.sqrt(wl.head_dim)})
        work.append(int(lens[ss].sum()) * wl.num_kv_heads * wl.head_dim * 4)
    return tasks, work


def prefill_tasks(batch, wl, n: int, paged: bool):
    """Causal prefill of every sequence, split in n shares: packed q/k/v slices, or (paged) the
    queries with a host copy of the blocks their tables name (the new tokens already stored)."""
    from tests.parity import Compact  # test infrastructure, used only for this leg
    from workloads import tensors

    q = tensors.to_u16(batch.q)
    k = v = None
    if not paged:
        k, v = tensors.to_u16(batch.k_new), tensors.to_u16(batch.v_new)
    cq, ck = wl.cu_seqlens_q.astype(np.int64), wl.cu_seqlens_k.astype(np.int64)
    nq, nk = np.diff(cq), np.diff(ck)
    pairs = [int((b - a) * a + a * (a + 1) // 2) for a, b in zip(nq, nk)]
    tasks, work = [], []
    for share in balanced_shares(pairs, n):
        rows = np.concatenate([np.arange(cq[i], cq[i + 1]) for i in share])
        cu_q = np.concatenate([[0], np.cumsum(nq[share])]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(nk[share])]).astype(np.int32)
        task = {"kind": "prefill", "q": q[rows], "cu_q": cu_q, "cu_k": cu_k, "scale": 1.0 / math.sqrt(wl.head_dim)}
        if paged:
            host = Compact(batch, share)
            task.update(k=host.k, v=host.v, tables=host.tables)
        else:
            krows = np.concatenate([np.arange(ck[i], ck[i + 1]) for i in share])
            task.update(k=k[krows], v=v[krows])
        tasks.append(task)
        work.append(sum(pairs[i] for i in share) * 4 * wl.head_dim * wl.num_q_heads)
    return tasks, work


def run_oracle_baseline(pool, tasks, work, unit: str, sample: str) -> dict:
    secs = pool.map(_oracle_worker, tasks, chunksize=1)
    total, slowest = float(sum(work)), max(secs)
    scale = 1e9 if unit == "GB/s" else 1e12
    return {"value": total / slowest / scale, "unit": unit, "cores": len(tasks), "kind": "oracle",
            "host_cores_available": host_cores(), "host_cpu_count": os.cpu_count(),
            "oracle_s_slowest_share": round(slowest, 3), "oracle_s_all_shares": round(float(sum(secs)), 3),
            "sample": sample + f"; numpy fp64, {len(tasks)} worker processes with one BLAS thread each"}


def cpu_baselines(pool, n, b2, wl2, b3, wl3, b4, wl4, b5, wl5, long_sample: int = 128) -> dict:
    """Oracle baselines for the decode, prefill, prefix and long-decode batches (each leg's own unit)."""
    res = {}
    tasks, work = decode_tasks(b2, wl2, list(range(wl2.num_seqs)), n)
    res["cpu_baseline"] = run_oracle_baseline(
        pool, tasks, work, "GB/s", f"store + decode of all {wl2.num_seqs} sequences of the decode batch "
        f"({sum(work) / 1e9:.3f} GB of K/V)")
    tasks, work = prefill_tasks(b3, wl3, n, paged=False)
    res["cpu_baseline_prefill"] = run_oracle_baseline(
        pool, tasks, work, "TFLOP/s", f"causal prefill of all {wl3.num_seqs} sequences of the varlen batch "
        f"({sum(work) / 1e9:.2f} GFLOP of unmasked pairs)")
    tasks, work = prefill_tasks(b4, wl4, n, paged=True)
    res["cpu_baseline_prefix_prefill"] = run_oracle_baseline(
        pool, tasks, work, "TFLOP/s", f"prefix-cached prefill of all {wl4.num_seqs} sequences through their "
        f"block tables ({sum(work) / 1e9:.2f} GFLOP of unmasked pairs)")
    if b5 is not None:
        seqs = sorted(np.random.default_rng(505).choice(wl5.num_seqs, min(long_sample, wl5.num_seqs),
                                                        replace=False).tolist())
        tasks, work = decode_tasks(b5, wl5, seqs, n)
        res["cpu_baseline_long_decode"] = run_oracle_baseline(
            pool, tasks, work, "GB/s", f"store + decode of {len(seqs)} of the {wl5.num_seqs} long-context "
            f"sequences, drawn uniformly with seed 505 ({sum(work) / 1e9:.3f} GB of K/V)")
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--split-waves", type=int, default=0, help="decode work split (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-decode", action="store_true",
                    help="leave the long-context decode leg (161 GiB pool, about 14 GB of K/V per step) out of the step")
    ap.add_argument("--step-only", action="store_true",
                    help="skip the untimed host block-manager, decode-graph and cold-launch legs (profiling runs)")
    ap.add_argument("--decode-graph-only", action="store_true",
                    help="run only the eager-vs-graph decode-step leg and print its JSON (for a kernel trace of it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run one 256 MiB device copy (reads and writes a known byte count) "
                         "so that profiler byte counters can be calibrated against it")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this build measures one GPU only; the path is data-parallel and shards by "
                                   "sequence or kv head with no exchange, so run one process per GPU",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    if args.decode_graph_only:
        import torch

        import paged_kv_cache_heads_amd as pa
        from workloads import configs, tensors
        wl2 = configs.config2()
        b2 = tensors.materialize(wl2, torch.device("cuda:0"))
        print(json.dumps({"decode_graph": decode_graph_latency(pa, torch, b2, wl2, 1.0 / math.sqrt(128))}),
              flush=True)
        return
    # the oracle's worker processes start before anything touches the GPU
    n_cores = host_cores()
    pool = None if args.no_cpu_baseline else start_oracle_pool(n_cores)
    try:
        result = run(args, pool, n_cores)
    finally:
        if pool is not None:
            pool.terminate()
            pool.join()
    print(json.dumps(result), flush=True)


def run(args, pool, n_cores) -> dict:
    import torch

    import paged_kv_cache_heads_amd as pa
    from workloads import configs, tensors

    dev = torch.device("cuda:0")
    pa._lib.load()
    scale = 1.0 / math.sqrt(128)

    wl2, wl3, wl4 = configs.config2(), configs.config3(), configs.config4()
    b2 = tensors.materialize(wl2, dev)
    b3 = tensors.materialize(wl3, dev)
    b4 = tensors.materialize(wl4, dev)
    ws_bytes = pa.pa_decode_workspace_size(wl2.num_seqs, 16, 8, 128, wl2.max_context_len, args.split_waves)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    out2 = torch.empty((wl2.num_seqs, 16, 128), dtype=torch.bfloat16, device=dev)
    out3 = torch.empty((wl3.num_tokens, 16, 128), dtype=torch.bfloat16, device=dev)
    out4 = torch.empty((wl4.num_tokens, 16, 128), dtype=torch.bfloat16, device=dev)
    mq3, mq4, mk2 = wl3.max_seqlen_q, wl4.max_seqlen_q, wl2.max_context_len
    # long-context batch: the pool is 60% of HBM for one layer's K and V; rows no sequence holds are
    # zero-filled (the parity tests fill them with NaN), to keep the set-up short
    wl5 = b5 = ws5 = out5 = None
    if not args.no_long_decode:
        wl5 = configs.config5()
        b5 = tensors.materialize(wl5, dev, fill_nan=False)
        mk5 = wl5.max_context_len
        ws5 = torch.empty(max(pa.pa_decode_workspace_size(wl5.num_seqs, 32, 8, 128, mk5, args.split_waves), 16),
                          dtype=torch.uint8, device=dev)
        out5 = torch.empty((wl5.num_seqs, 32, 128), dtype=torch.bfloat16, device=dev)
    from workloads import rope
    nr_rng = np.random.default_rng(7)
    nr_qw = torch.as_tensor(rope.norm_weight(nr_rng, 128).view(np.int16)).to(dev).view(torch.bfloat16)
    nr_kw = torch.as_tensor(rope.norm_weight(nr_rng, 128).view(np.int16)).to(dev).view(torch.bfloat16)
    nr_table = torch.as_tensor(rope.cos_sin_table(40960, 128, base=1.0e6)).to(dev)
    nr_pos = torch.as_tensor(wl3.store_pos.astype(np.int32)).to(dev)
    nr_q = torch.empty((wl3.num_tokens, 16, 128), dtype=torch.bfloat16, device=dev)
    # sampler: one token per decode sequence over a 151936-token vocabulary (fp32 logits, N(0, 2^2))
    smp_gen = torch.Generator(device=dev)
    smp_gen.manual_seed(9)
    smp_logits = torch.randn((wl2.num_seqs, SAMPLER_VOCAB), generator=smp_gen, device=dev) * 2.0
    smp_temps = torch.full((wl2.num_seqs,), 0.8, dtype=torch.float32, device=dev)
    smp_tokens = torch.empty(wl2.num_seqs, dtype=torch.int32, device=dev)
    smp_ws = torch.empty(pa.pa_sample_workspace_size(wl2.num_seqs, SAMPLER_VOCAB), dtype=torch.uint8, device=dev)

    kernels = ["decode", "long_decode", "store_prefill", "prefill", "store_prefix", "prefill_prefix",
               "norm_rope_prefill", "sample_decode"]
    if b5 is None:
        kernels.remove("long_decode")
    calls = {
        "decode": lambda: pa.pa_store_decode(b2.q, b2.k_new, b2.v_new, b2.k_cache, b2.v_cache, b2.block_tables,
                                             b2.context_lens, scale, mk2, out=out2, workspace=ws,
                                             split_waves=args.split_waves),
        "long_decode": lambda: pa.pa_store_decode(b5.q, b5.k_new, b5.v_new, b5.k_cache, b5.v_cache,
                                                  b5.block_tables, b5.context_lens, scale, wl5.max_context_len,
                                                  out=out5, workspace=ws5, split_waves=args.split_waves),
        "store_prefill": lambda: pa.pa_store_kvcache(b3.k_new, b3.v_new, b3.k_cache, b3.v_cache, b3.slot_mapping),
        "prefill": lambda: pa.pa_prefill_varlen(b3.q, b3.k_new, b3.v_new, b3.cu_seqlens_q, b3.cu_seqlens_k, mq3,
                                                wl3.max_seqlen_k, scale, out=out3),
        "store_prefix": lambda: pa.pa_store_kvcache(b4.k_new, b4.v_new, b4.k_cache, b4.v_cache, b4.slot_mapping),
        "prefill_prefix": lambda: pa.pa_prefill_varlen(b4.q, b4.k_cache, b4.v_cache, b4.cu_seqlens_q,
                                                       b4.cu_seqlens_k, mq4, wl4.max_seqlen_k, scale,
                                                       block_table=b4.block_tables, out=out4),
        "norm_rope_prefill": lambda: pa.pa_qk_norm_rope_store(b3.qkv, nr_qw, nr_kw, 1e-6, nr_table, nr_pos,
                                                              b3.k_cache, b3.v_cache, b3.slot_mapping, 16,
                                                              q_out=nr_q),
        "sample_decode": lambda: pa.pa_sample_gumbel(smp_logits, smp_temps, 1234, 0, tokens=smp_tokens,
                                                     workspace=smp_ws),
    }

    def step(events=None, i=0):
        for n, name in enumerate(kernels):
            if events is not None:
                events[i][n][0].record()
            calls[name]()
            if events is not None:
                events[i][n][1].record()

    # events and the lead-in are set up before the warm-up steps, so that the timed steps follow them
    # without an idle gap (the clocks of MFMA-bound launches ramp up again over ~10 ms after one)
    ev = [[(TimingEvent(), TimingEvent()) for _ in kernels]
          for _ in range(args.steps)]
    lead = lead_in_cycles(torch)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # The queue is empty here, so without a lead-in the first leg's start event of the first step would
    # fire at once and its duration would include the host's own launch path (30-100 us measured, against
    # under 2 us once the host runs ahead). A spin of about LEAD_IN_US keeps the queue busy while the host
    # enqueues that step; it is inside the timed region, so ms_per_step includes it.
    torch.cuda._sleep(lead)
    for i in range(args.steps):
        step(ev, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {name: float(np.mean([ev[i][n][0].elapsed_time(ev[i][n][1]) for i in range(args.steps)]))
          for n, name in enumerate(kernels)}
    stats = {}
    for n, name in enumerate(kernels):
        t = [ev[i][n][0].elapsed_time(ev[i][n][1]) * 1e3 for i in range(args.steps)]
        stats[name] = {"median": round(float(np.median(t)), 2), "min": round(float(np.min(t)), 2),
                       "max": round(float(np.max(t)), 2)}
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    peaks = measured_peaks(torch, dev)
    # after the timed steps: each launch alone with the caches flushed first (a 512 MiB write, untimed);
    # skipped in profiling runs, whose per-kernel statistics cover the timed steps only
    cold, cold_stats = (None, None) if args.step_only else cold_launches(torch, dev, kernels, calls)

    # Each roofline also gives the launch's cold figure (run alone right after a 512 MiB write has flushed
    # L2 and MALL), the timing the protocol asks for where the working set fits in those caches.
    def cold_fields(leg: str, work: float, peak: float) -> dict:
        if not cold:
            return {}
        return {"cold_launch_us": cold[leg], "frac_cold": round(work / (cold[leg] * 1e-6) / peak, 4)}

    def hbm_roofline(kernel: str, leg: str, nbytes: int, traffic=None, **extra):
        gbs = nbytes / (ms[leg] * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "bytes_per_launch": nbytes,
                "avg_launch_us": round(ms[leg] * 1e3, 2), **cold_fields(leg, nbytes / 1e9, HBM_PEAK_GBS), **extra}

    def mfma_roofline(kernel: str, leg: str, flops: int):
        tf = flops / (ms[leg] * 1e-3) / 1e12
        return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "frac_of_measured_gemm": round(tf / peaks["bf16_gemm_TFLOPs"], 4), "flops_per_launch": flops,
                "avg_launch_us": round(ms[leg] * 1e3, 2), **cold_fields(leg, flops / 1e12, MFMA_BF16_PEAK_TFLOPS)}

    dbytes = decode_bytes(wl2)
    leg_bytes = dbytes["total"] + store_bytes(wl2, wl2.num_seqs)  # the decode plus the new tokens' store
    value = dbytes["kv"] / (ms["decode"] * 1e-3) / 1e9
    f3, f4 = prefill_flops(wl3), prefill_flops(wl4)
    nrb = norm_rope_bytes(wl3, wl3.num_tokens)
    smp_bytes = wl2.num_seqs * (SAMPLER_VOCAB * 4 + 4 + 4)
    sb = {"store_prefill": store_bytes(wl3, wl3.num_tokens), "store_prefix": store_bytes(wl4, wl4.num_tokens)}
    workload = ("decode step of 256 seqs, context U{100..2048} (Hq 16, Hkv 8, D 128, 256-token blocks, "
                "4096-block pool)")
    if b5 is not None:
        workload += (" + long-context decode step of 512 seqs, context log-uniform 256..32768 (Hq 32, Hkv 8, "
                     "164,794-block pool)")
    workload += (" + varlen causal prefill (%d seqs, %d tokens) + prefix-cached prefill (32 seqs, 1024 shared + "
                 "%d new tokens)" % (wl3.num_seqs, wl3.num_tokens, wl4.num_tokens))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "lead_in_us": LEAD_IN_US,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "value_is": "KV-read GB/s of the 256-sequence decode leg (K and V bytes of every context token over "
                        "the leg's event time)",
            "decode_kv_bytes": dbytes["kv"],
            "decode_split_waves": pa.pa_decode_split_waves(wl2.num_seqs, 16, 8, mk2, args.split_waves),
            "prefill_flops": f3,
            "prefix_prefill_flops": f4,
        },
        "pages_end_to_end_context": PAGES_END_TO_END,
        "roofline": hbm_roofline("pa_store_decode (split kernel with the store fused + finalize)", "decode",
                                 leg_bytes, measured_traffic("decode")),
        "roofline_prefill": mfma_roofline("prefill_kernel (varlen, packed)", "prefill", f3),
        "roofline_prefix_prefill": mfma_roofline("prefill_kernel (block table)", "prefill_prefix", f4),
        "roofline_norm_rope_store": hbm_roofline("norm_rope_store_kernel (varlen prefill batch)",
                                                 "norm_rope_prefill", nrb),
        "roofline_sampler": hbm_roofline("sample_partial + sample_final (256 x 151936 fp32 logits)",
                                         "sample_decode", smp_bytes),
        "roofline_store": {k: hbm_roofline("store_tokens_kernel (%s batch)" % (
                               "varlen" if k == "store_prefill" else "prefix"), k, sb[k],
                               frac_of_measured_copy=round(sb[k] / (ms[k] * 1e-3) / 1e9 / peaks["copy_GBs"], 4))
                           for k in sb},
        "kernels_us": {k: round(v * 1e3, 2) for k, v in ms.items()},
        "kernels_us_stats": stats,
        "kernels_us_cold": cold,
        "kernels_us_cold_stats": cold_stats,
        "measured_peaks": peaks,
    }
    if b5 is not None:
        d5 = decode_bytes(wl5)
        result["config"]["long_decode_kv_bytes"] = d5["kv"]
        result["config"]["long_decode_split_waves"] = pa.pa_decode_split_waves(wl5.num_seqs, 32, 8,
                                                                               wl5.max_context_len, args.split_waves)
        result["roofline_long_decode"] = hbm_roofline(
            "pa_store_decode (split kernel with the store fused + finalize), long-context batch", "long_decode",
            d5["total"] + store_bytes(wl5, wl5.num_seqs), measured_traffic("long_decode"),
            kv_GBs=round(d5["kv"] / (ms["long_decode"] * 1e-3) / 1e9, 1))
    if not args.step_only:
        result["decode_separate_calls"] = separate_decode_leg(pa, torch, b2, wl2, scale, mk2, ws, out2, args.steps,
                                                              args.warmup, args.split_waves)
        if b5 is not None:
            result["long_decode_separate_calls"] = separate_decode_leg(
                pa, torch, b5, wl5, scale, wl5.max_context_len, ws5, out5, args.steps, args.warmup, args.split_waves)
        result["store_references"] = store_references(pa, torch, b3, wl3)
        result["store_prefill_fused"] = fused_store_prefill(pa, torch, scale, b3, wl3, b4, wl4, out3, out4)
        result["host_block_manager"] = host_block_manager(wl2, wl4)
        result["decode_graph"] = decode_graph_latency(pa, torch, b2, wl2, scale)
    if pool is not None:
        result.update(cpu_baselines(pool, n_cores, b2, wl2, b3, wl3, b4, wl4, b5, wl5))
    return result


if __name__ == "__main__":
    main()
