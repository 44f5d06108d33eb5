"""Graph-captured decode steps (pa_decode_graphs_*) against the eager step and the oracle.

Graphs hold pa_store_decode, captured once for batch sizes 1, 2, 4, ..., 512 over fixed buffers,
and take the live batch from a device int32. For several real batch sizes the first rows are
filled (ordinary eager work) and the rows past the batch are left holding garbage: stale lengths,
and block tables that name a canary block. The graph of the next size up is replayed. Its output
rows must equal, bit for bit, the eager pa_store_decode launched at the padded size with zero
lengths past the batch (the launch size sets the work split). The rows past the batch must come
out zero, and the canary block must stay untouched. Every size is replayed several times with
eager work and synchronisation in between, each replay checked. One case is also checked against
the oracle.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_heads_amd as pa
from tests.gpu_common import announce, dev  # noqa: F401
from tests.parity import Compact, assert_attention_close
from workloads import configs, tensors

pytestmark = pytest.mark.gpu

SIZES = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512]


@pytest.mark.parametrize("hq", [16, 64])
def test_decode_graphs_match_eager_and_oracle(dev, hq):
    # 16 query heads: the vector split pass; 64 (8 per kv head): the matrix-core split pass
    announce(f"decode graphs 1..512 vs eager, {hq} query heads")
    if hq == 16:
        wl = configs.config2()  # 256 sequences, L ~ U{100..2048}, 4096-block pool (about 1200 used)
    else:
        lens = np.random.default_rng([2, 0]).integers(100, 2048, size=256, endpoint=True)
        wl = configs.decode_workload("cfg2-g8", lens, hq, 8, 4096, 2)
    b = tensors.materialize(wl, dev)
    scale = 1.0 / math.sqrt(128)
    w = int(b.block_tables.shape[1])
    maxb = SIZES[-1]
    max_len = w * wl.block_size
    canary = wl.num_blocks - 1  # a block no sequence of the batch uses
    assert canary not in set(wl.block_tables.ravel().tolist())
    # the step's fixed buffers
    q_s = torch.randn((maxb, hq, 128), device=dev).to(torch.bfloat16)
    k_s = torch.randn((maxb, 8, 128), device=dev).to(torch.bfloat16)
    v_s = torch.randn((maxb, 8, 128), device=dev).to(torch.bfloat16)
    bt_s = torch.full((maxb, w), canary, dtype=torch.int32, device=dev)
    cl_s = torch.full((maxb,), 777, dtype=torch.int32, device=dev)  # stale lengths past every batch
    out_s = torch.empty((maxb, hq, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(pa.pa_decode_workspace_size(maxb, hq, 8, 128, max_len), dtype=torch.uint8, device=dev)
    canary_k, canary_v = b.k_cache[canary].clone(), b.v_cache[canary].clone()
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        graphs = pa.DecodeGraphs(q_s, k_s, v_s, bt_s, cl_s, out_s, ws, b.k_cache, b.v_cache, scale, max_len,
                                 SIZES)
        ws_e = torch.empty(pa.pa_decode_workspace_size(maxb, hq, 8, 128, max_len), dtype=torch.uint8, device=dev)
        checked_oracle = False
        for batch in (1, 3, 17, 100, 255, 256):
            rows = torch.arange(batch, device=dev)
            padded = min(s for s in SIZES if s >= batch)
            for rep in range(3):
                # eager work between replays: fill the step's rows and the live count
                q_s[:batch] = b.q[rows]
                k_s[:batch] = b.k_new[rows]
                v_s[:batch] = b.v_new[rows]
                bt_s[:batch] = b.block_tables[rows]
                cl_s[:batch] = b.context_lens[rows]
                graphs.live_batch.fill_(batch)
                out_s.fill_(1.0)
                got_padded = graphs.launch(batch, live_written=(rep != 1))
                stream.synchronize()
                assert got_padded == padded
                got = out_s[:batch].clone()
                assert torch.all(out_s[batch:padded].float() == 0)
                for cache, saved in ((b.k_cache, canary_k), (b.v_cache, canary_v)):  # bits (the block holds NaN)
                    assert torch.equal(cache[canary].view(torch.int16), saved.view(torch.int16))
                # the eager step at the padded size, lengths past the batch zero (same work split)
                cl_e = cl_s[:padded].clone()
                cl_e[batch:] = 0
                ref = pa.pa_store_decode(q_s[:padded], k_s[:padded], v_s[:padded], b.k_cache, b.v_cache,
                                         bt_s[:padded], cl_e, scale, max_len, workspace=ws_e)
                stream.synchronize()
                assert torch.equal(got.view(torch.int16), ref[:batch].view(torch.int16)), (batch, rep)
            if batch == 17 and not checked_oracle:
                seqs = list(range(batch))
                host = Compact(b, seqs)  # the new tokens are in the cache already (stored by the replays)
                want = oracle.decode(tensors.to_u16(b.q[:batch]), host.k, host.v, host.tables,
                                     wl.context_lens[:batch], scale)
                assert_attention_close(got, want, f"graph decode, 17 sequences, {hq} query heads")
                checked_oracle = True
        graphs.close()


def test_decode_graphs_reject_bad_arguments(dev):
    announce("decode graphs argument errors")
    wl = configs.config1()
    b = tensors.materialize(wl, dev)
    maxb = 4
    w = int(b.block_tables.shape[1])
    bufs = [torch.zeros((maxb, 16, 128), dtype=torch.bfloat16, device=dev),
            torch.zeros((maxb, 8, 128), dtype=torch.bfloat16, device=dev),
            torch.zeros((maxb, 8, 128), dtype=torch.bfloat16, device=dev),
            torch.full((maxb, w), -1, dtype=torch.int32, device=dev),
            torch.zeros((maxb,), dtype=torch.int32, device=dev),
            torch.empty((maxb, 16, 128), dtype=torch.bfloat16, device=dev)]
    small_ws = torch.empty(16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        with pytest.raises(pa.PAError):  # not increasing
            pa.DecodeGraphs(*bufs, small_ws, b.k_cache, b.v_cache, 0.1, w * 256, [2, 2])
        with pytest.raises(pa.PAError) as e:  # workspace too small: the captured decode's own status
            pa.DecodeGraphs(*bufs, small_ws, b.k_cache, b.v_cache, 0.1, w * 256, [1, 4])
        assert e.value.status == 5
        ws = torch.empty(pa.pa_decode_workspace_size(maxb, 16, 8, 128, w * 256), dtype=torch.uint8, device=dev)
        g = pa.DecodeGraphs(*bufs, ws, b.k_cache, b.v_cache, 0.1, w * 256, [1, 4])
        with pytest.raises(pa.PAError):
            g.launch(5)
        with pytest.raises(pa.PAError):
            g.launch(0)
        g.close()
