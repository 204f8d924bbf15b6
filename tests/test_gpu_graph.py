"""The resolver and the decode captured once in a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay must match the oracle exactly (the resolver) or the
eager call (the decode).  Between replays the test does eager work of its own:
the forward pass's row writes and the next step's inputs copied into the
graph's static buffers.  The library's stream entry points only launch kernels
on the given stream (no allocation, memset or synchronisation once the pool and
the decode workspace exist), which is what makes them capturable
("vLLM HiSparse 本地 KV 卸载架构": graph-stable row IDs, no readback)."""
import math

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from tests.harness import Pair, make_host_pools
from workloads import fill_host_rows_mla, make_queries, synth

pytestmark = pytest.mark.gpu


def _workload():
    # 10 batch rows (the fused plan + copy instance runs at batch >= 8): long
    # rows on the LRU path, two fast-path rows, resident tail pages, one
    # padding row.
    return synth("graph", 41, R=10, S=256, k=96, steps=7,
                 n0=[3000, 2500, 900, 4000, 200, 5000, 1200, 3500, 2800, 150], grow=1,
                 keep=70, recent=8, recent_window=128, P=16, resident_tail=64, padding_rows=1)


@pytest.mark.parametrize("mode", ["resolve", "split"])
def test_resolver_replayed_from_a_graph(mode):
    print("[graph] resolver mode=%s" % mode, flush=True)
    w = _workload()
    pair = Pair(w, make_host_pools(w, kind="uniform"), mode=mode)
    try:
        dst, src = pair.gpu_step(0)  # eager first step (and warm-up)
        o = pair.oracle_step(0, dst, src)
        torch.cuda.synchronize()
        pair.compare_step(0, o)

        topk_s = pair.topk[1].clone()
        seq_s = pair.seq[1].clone()
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            args = (pair.pool, None, w.B, w.k, pair.req_idx, topk_s, seq_s, pair.locs, pair.bt,
                    pair.st, pair.lru, pair.clk, pair.out, pair.stats)
            if mode == "resolve":
                hs.hisparse_resolve(*args)
            else:
                hs.hisparse_resolve_plan(*args)
                hs.hisparse_gather_copy(pair.pool, None, w.B, 0, w.L, pair.stats)
        torch.cuda.synchronize()

        for step in range(1, w.steps):
            dst, src = pair.pre_step_writes(step)
            topk_s.copy_(pair.topk[step])
            seq_s.copy_(pair.seq[step])
            graph.replay()
            o = pair.oracle_step(step, dst, src)
            torch.cuda.synchronize()
            pair.compare_step(step, o)
            print("[graph] replay of step %d matches the oracle" % step, flush=True)
        pair.compare_pools()
    finally:
        pair.close()


def test_decode_replayed_from_a_graph():
    print("[graph] decode", flush=True)
    B, H, k, rows = 6, 128, 700, 2000
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 8, gen_device="cuda")
    rng = np.random.default_rng(8)
    locs_np = rng.integers(-1, rows, size=(B, k)).astype(np.int32)
    locs = torch.from_numpy(locs_np).cuda()
    hb = hs.HostBuffer(656 * 16)
    cfg = hs.PoolConfig(max_requests=1, slots=k, max_top_k=k, max_batch=B, max_seq_len=16)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], rows)
    scale = 1.0 / math.sqrt(192.0)
    try:
        qs = [make_queries(B, H, seed=30 + t, device="cuda") for t in range(3)]
        want = []
        for q in qs:  # eager calls (the first one also sizes the split workspace)
            o = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
            hs.hisparse_sparse_mla_decode(pool, None, B, H, k, 0, q, locs, scale, o)
            want.append(o)
        torch.cuda.synchronize()

        q_s = qs[0].clone()
        out_s = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            hs.hisparse_sparse_mla_decode(pool, None, B, H, k, 0, q_s, locs, scale, out_s)
        torch.cuda.synchronize()

        for rep in range(2):
            for t, q in enumerate(qs):
                q_s.copy_(q)
                out_s.zero_()
                graph.replay()
                torch.cuda.synchronize()
                assert torch.equal(out_s, want[t]), "replay %d of query set %d differs" % (rep, t)
        print("[graph] 6 decode replays equal the eager calls", flush=True)
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


def test_overlapped_layers_replayed_from_a_graph():
    """Plan plus the overlapped per-layer copy and decode (two pool streams
    forked from the caller's stream by events and joined back) captured once
    and replayed: each replay equals the eager sequential order bit for bit
    (row IDs, state, counters, device pools, every layer's output)."""
    print("[graph] overlapped layers", flush=True)
    B, L, H = 9, 3, 32
    scale = 1.0 / math.sqrt(192.0)
    w = synth("ovlgraph", 91, R=B, S=256, k=128, steps=5, n0=[3000 + 700 * b for b in range(B)],
              L=L, grow=1, keep=80, recent=16, recent_window=64)
    bufs = make_host_pools(w, kind="mla")
    seq = Pair(w, bufs, with_oracle=False)
    ovl = Pair(w, bufs, with_oracle=False)
    try:
        qs = [make_queries(w.B, H, seed=20 + l, device="cuda") for l in range(L)]
        outs_s = [torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        outs_o = [torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        topk_s = ovl.topk[0].clone()
        seq_s = ovl.seq[0].clone()

        def sequential(step):
            seq.pre_step_writes(step)
            hs.hisparse_resolve_plan(seq.pool, None, w.B, w.k, seq.req_idx, seq.topk[step],
                                     seq.seq[step], seq.locs, seq.bt, seq.st, seq.lru, seq.clk,
                                     seq.out, seq.stats)
            hs.hisparse_gather_copy(seq.pool, None, w.B, 0, L, seq.stats)
            for l in range(L):
                hs.hisparse_sparse_mla_decode(seq.pool, None, w.B, H, w.k, l, qs[l], seq.out, scale,
                                              outs_s[l])

        def overlapped():
            hs.hisparse_resolve_plan(ovl.pool, None, w.B, w.k, ovl.req_idx, topk_s, seq_s, ovl.locs,
                                     ovl.bt, ovl.st, ovl.lru, ovl.clk, ovl.out, ovl.stats)
            hs.hisparse_decode_layers_overlapped(ovl.pool, None, w.B, H, w.k, qs, ovl.out, scale,
                                                 outs_o, ovl.stats)

        def compare(step):
            torch.cuda.synchronize()
            assert torch.equal(seq.out, ovl.out), "row IDs, step %d" % step
            for a, b in ((seq.st, ovl.st), (seq.lru, ovl.lru), (seq.clk, ovl.clk),
                         (seq.stats, ovl.stats)):
                assert torch.equal(a, b), "state, step %d" % step
            for l in range(L):
                assert torch.equal(seq.dev_pools[l], ovl.dev_pools[l]), "pool %d, step %d" % (l, step)
                assert torch.equal(outs_s[l], outs_o[l]), "output of layer %d, step %d" % (l, step)

        # step 0 eagerly on both sides: it also creates the pool's streams,
        # events and decode workspace, which capture cannot
        sequential(0)
        ovl.pre_step_writes(0)
        overlapped()
        compare(0)

        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            overlapped()
        torch.cuda.synchronize()

        for step in range(1, w.steps):
            sequential(step)
            ovl.pre_step_writes(step)
            topk_s.copy_(ovl.topk[step])
            seq_s.copy_(ovl.seq[step])
            graph.replay()
            compare(step)
            print("[graph] overlapped replay of step %d equals the sequential order" % step, flush=True)
    finally:
        seq.close()
        ovl.close()
