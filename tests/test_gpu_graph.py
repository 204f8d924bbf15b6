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
    cfg = hs.PoolConfig(max_requests=1, slots=k, max_top_k=k, max_batch=B, max_seq_len=16,
                        max_heads=H)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], rows)
    scale = 1.0 / math.sqrt(192.0)
    try:
        qs = [make_queries(B, H, seed=30 + t, device="cuda") for t in range(3)]
        # The pool's first decode call is the captured one: the split
        # workspace was sized at init, so nothing needs allocating.
        q_s = qs[0].clone()
        out_s = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            hs.hisparse_sparse_mla_decode(pool, None, B, H, k, 0, q_s, locs, scale, out_s)
        torch.cuda.synchronize()

        want = []
        for q in qs:  # eager calls on the same pool
            o = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
            hs.hisparse_sparse_mla_decode(pool, None, B, H, k, 0, q, locs, scale, o)
            want.append(o)
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


def test_noalloc_decode_replayed_from_a_graph():
    """The allocation-free decode captured in a graph (after one eager call,
    which looks up its static workspace on this device) and replayed over
    three query sets, twice: every replay equals the eager call."""
    print("[graph] allocation-free decode", flush=True)
    B, H, k, rows = 5, 144, 600, 1500
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 9, gen_device="cuda")
    rng = np.random.default_rng(9)
    locs = torch.from_numpy(rng.integers(-1, rows, size=(B, k)).astype(np.int32)).cuda()
    scale = 1.0 / math.sqrt(192.0)
    qs = [make_queries(B, H, seed=40 + t, device="cuda") for t in range(3)]
    want = []
    for q in qs:
        o = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
        hs.hisparse_sparse_mla_decode_noalloc(None, B, H, k, dev, q, locs, scale, o)
        want.append(o)
    torch.cuda.synchronize()
    q_s = qs[0].clone()
    out_s = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        hs.hisparse_sparse_mla_decode_noalloc(None, B, H, k, dev, q_s, locs, scale, out_s)
    torch.cuda.synchronize()
    for rep in range(2):
        for t, q in enumerate(qs):
            q_s.copy_(q)
            out_s.zero_()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out_s, want[t]), "replay %d of query set %d differs" % (rep, t)
            # an eager call between replays, on the same static workspace
            o = torch.empty_like(out_s)
            hs.hisparse_sparse_mla_decode_noalloc(None, B, H, k, dev, qs[(t + 1) % 3], locs, scale, o)
            torch.cuda.synchronize()
            assert torch.equal(o, want[(t + 1) % 3])
    print("[graph] 6 allocation-free decode replays equal the eager calls", flush=True)


def test_overlapped_layers_replayed_from_a_graph():
    """Plan plus the overlapped per-layer copy and decode (every launch on
    the caller's stream) captured once, before the pool has run anything,
    and replayed: each replay equals the eager sequential order bit for bit
    (row IDs, state, counters, device pools, every layer's output)."""
    print("[graph] overlapped layers", flush=True)
    B, L, H = 9, 3, 32
    scale = 1.0 / math.sqrt(192.0)
    w = synth("ovlgraph", 91, R=B, S=256, k=128, steps=5, n0=[3000 + 700 * b for b in range(B)],
              L=L, grow=1, keep=80, recent=16, recent_window=64)
    bufs = make_host_pools(w, kind="mla")
    seq = Pair(w, bufs, with_oracle=False, max_heads=H)
    ovl = Pair(w, bufs, with_oracle=False, max_heads=H)
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

        # captured before the pool's first call: the decode workspace was
        # sized at init, so the first overlapped call allocates nothing
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            overlapped()
        torch.cuda.synchronize()

        for step in range(w.steps):
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


def test_steps_and_maintenance_replayed_from_a_graph():
    """Two verification steps, a row mirror, invalidation by token range and
    by host rows, captured once and replayed for five decode steps on one
    pool; an identical pool runs the same calls eagerly.  Every replay must
    leave both bit-identical: row IDs, state, counters, device pools and the
    mirrored host rows."""
    print("[graph] verification steps and maintenance", flush=True)
    Q, D, k, L, B = 2, 5, 64, 2, 9
    w = synth("stepsgraph", 93, R=B + 1, S=(Q + 1) * k, k=k, steps=Q * D,
              n0=[3000 + 500 * b for b in range(B)], L=L, grow=1, keep=k // 2, recent=k // 4,
              recent_window=2 * k)
    eager = Pair(w, make_host_pools(w), with_oracle=False, max_steps=Q)
    graphed = Pair(w, make_host_pools(w), with_oracle=False, max_steps=Q)
    rng = np.random.default_rng(93)
    try:
        r0 = int(w.req_idx[0])
        dev = torch.device("cuda")
        # per pair: static inputs and outputs of the captured calls
        st_in = {}
        for name, p in (("eager", eager), ("graphed", graphed)):
            st_in[name] = dict(
                topk=torch.empty((Q, w.B, w.k), dtype=torch.int32, device=dev),
                seq=torch.empty((Q, w.B), dtype=torch.int32, device=dev),
                out=torch.empty((Q, w.B, w.k), dtype=torch.int32, device=dev),
                mir_d=torch.empty(8, dtype=torch.int32, device=dev),
                mir_h=torch.empty(8, dtype=torch.int64, device=dev),
                inv_lo=torch.empty(w.B, dtype=torch.int32, device=dev),
                inv_hi=torch.empty(w.B, dtype=torch.int32, device=dev),
                inv_rows=torch.empty(16, dtype=torch.int64, device=dev))

        def calls(p, s):
            hs.hisparse_resolve_steps(p.pool, None, Q, w.B, w.k, p.req_idx, s["topk"], s["seq"],
                                      p.locs, p.bt, p.st, p.lru, p.clk, s["out"], p.stats)
            hs.hisparse_mirror_rows(p.pool, None, s["mir_d"], s["mir_h"], stats=p.stats)
            hs.hisparse_invalidate_tokens(p.pool, None, p.req_idx, s["inv_lo"], s["inv_hi"], p.st,
                                          p.lru, p.stats)
            hs.hisparse_invalidate_host_rows(p.pool, None, s["inv_rows"], p.locs, p.st, p.lru)

        def inputs(d):
            sl = slice(d * Q, (d + 1) * Q)
            n_last = w.seq_lens[d * Q + Q - 1]
            mir_d = np.array([r0 * w.S + (d * 8 + j) % w.S for j in range(8)], np.int32)
            mir_h = np.array([w.host_pool_rows - 1 - (d * 8 + j) for j in range(8)], np.int64)
            inv_lo = np.maximum(n_last - 40, 0).astype(np.int32)
            inv_hi = np.maximum(n_last - 30, 0).astype(np.int32)
            inv_rows = np.sort(rng.choice(w.host_pool_rows - 64, size=16, replace=False)).astype(np.int64)
            for name, p in (("eager", eager), ("graphed", graphed)):
                for q in range(Q):
                    p.pre_step_writes(d * Q + q)
                s = st_in[name]
                s["topk"].copy_(p.topk[sl])
                s["seq"].copy_(p.seq[sl])
                s["mir_d"].copy_(torch.from_numpy(mir_d))
                s["mir_h"].copy_(torch.from_numpy(mir_h))
                s["inv_lo"].copy_(torch.from_numpy(inv_lo))
                s["inv_hi"].copy_(torch.from_numpy(inv_hi))
                s["inv_rows"].copy_(torch.from_numpy(inv_rows))

        def compare(d):
            torch.cuda.synchronize()
            a, b = st_in["eager"], st_in["graphed"]
            assert torch.equal(a["out"], b["out"]), "row IDs, decode step %d" % d
            for x, y, what in ((eager.st, graphed.st, "slot_tokens"), (eager.lru, graphed.lru, "lru"),
                               (eager.clk, graphed.clk, "clock"), (eager.stats, graphed.stats, "stats")):
                assert torch.equal(x, y), "%s, decode step %d" % (what, d)
            for l in range(L):
                assert torch.equal(eager.dev_pools[l], graphed.dev_pools[l]), "pool %d" % l
                tail = slice(w.host_pool_rows - 64, w.host_pool_rows)
                assert np.array_equal(eager.host_np[l][tail], graphed.host_np[l][tail]), "host %d" % l

        inputs(0)
        calls(eager, st_in["eager"])
        calls(graphed, st_in["graphed"])   # eager warm-up of the graphed pool
        compare(0)

        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            calls(graphed, st_in["graphed"])
        torch.cuda.synchronize()

        for d in range(1, D):
            inputs(d)
            calls(eager, st_in["eager"])
            graph.replay()
            compare(d)
            print("[graph] decode step %d: replay equals the eager calls" % d, flush=True)
        assert int(graphed.stats[1].item()) > 0
    finally:
        eager.close()
        graphed.close()
