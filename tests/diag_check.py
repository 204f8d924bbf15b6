"""Checks of the diagnostic library (libhisparse_diag.so), run in a process of
its own with HISPARSE_LIBRARY=diag (the binding loads one library per
process): the build with the phase trace compiled in resolves bit-exactly like
the oracle, its trace is complete and ordered, and the floor kernels compute
what include/hisparse_diag.h states.  Prints "DIAG OK" at the end."""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

assert os.environ.get("HISPARSE_LIBRARY") == "diag", "run with HISPARSE_LIBRARY=diag"

import numpy as np  # noqa: E402
import torch  # noqa: E402

import hierarchical_sparse_attention_hisparse_amd as hs  # noqa: E402
from harness import Pair, make_host_pools, run_parity  # noqa: E402
from workloads import config1_tiny, config2_dsa_decode  # noqa: E402


def say(*a):
    print("[diag]", *a, flush=True)


def check_trace(tr, long_rows, other_rows):
    """Every wavefront of a long row passed points 0-7; the row's points are
    reached in order (last wavefront, real-time counter); other rows stop at
    point 0; the info point holds at most 4 windows and a 0/1 sort flag, the
    same in every wavefront."""
    for b in long_rows:
        t = tr[b]
        assert (t[:, :8, :] > 0).all(), "row %d: a phase point was not reached" % b
        last = t[:, :8, 1].astype(np.int64).max(axis=0)
        assert (np.diff(last) >= 0).all(), ("row %d: points out of order" % b, last)
        assert t[0, 8, 0] <= 4 and t[0, 8, 1] in (0, 1), ("row %d: ranking info" % b, t[0, 8])
        assert (t[:, 8, :] == t[0, 8, :]).all(), "row %d: wavefronts disagree on the ranking" % b
    for b in other_rows:
        assert (tr[b, :, 1:8, :] == 0).all(), "row %d (fast path): points past 0 written" % b
        assert (tr[b, :, 0, :] > 0).all(), "row %d: entry not recorded" % b


def main():
    assert hs.is_diag_library() and hs.library_path().endswith("libhisparse_diag.so")
    torch.cuda.set_device(0)

    # 1. parity of the traced build: tiny workload through both entry paths
    w1 = config1_tiny(steps=8)
    for mode in ("resolve", "split"):
        run_parity(w1, mode=mode)
        say("config1 8 steps bit-exact (%s)" % mode)

    # 2. DSA decode, fused (batch 72): parity and the trace of every step
    w2 = config2_dsa_decode(steps=3)
    bufs = make_host_pools(w2, "uniform")
    for mode in ("resolve", "split"):
        pair = Pair(w2, bufs, mode=mode)
        try:
            for step in range(w2.steps):
                hs.hisparse_diag_phase_clear()
                dst, src = pair.gpu_step(step)
                o_out = pair.oracle_step(step, dst, src)
                torch.cuda.synchronize()
                pair.compare_step(step, o_out)
                tr = hs.hisparse_diag_phase_read()
                long_rows = np.nonzero(w2.seq_lens[step] > w2.S)[0]
                other = np.nonzero(w2.seq_lens[step] <= w2.S)[0]
                assert len(long_rows) == 64 and len(other) == 8
                check_trace(tr, long_rows, other)
                assert (tr[w2.B:] == 0).all(), "rows past the batch written"
            pair.compare_pools()
        finally:
            pair.close()
        say("config2 3 steps bit-exact with a complete trace (%s)" % mode)

    # 3. floor kernels against their stated results
    dev = torch.device("cuda")
    g = torch.Generator().manual_seed(7)
    B, k, S, R, n = 9, 1500, 700, 5, 3000
    req = torch.tensor([0, 4, -3, 9, 2, 2, 1, 3, 4], dtype=torch.int32)
    topk = torch.randint(-5, n + 50, (B, k), generator=g, dtype=torch.int32)
    st = torch.randint(-2, n, (R, S), generator=g, dtype=torch.int32)
    lru = torch.randint(0, 1 << 30, (R, S), generator=g, dtype=torch.int32)
    locs = torch.randint(-(1 << 40), 1 << 40, (R, n), generator=g, dtype=torch.int64)
    out = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    d = lambda x: x.to(dev)
    hs.hisparse_diag_floor(None, 0, B, launches=3)
    hs.hisparse_diag_floor(None, 1, B, k, S, R, n, d(req), None, None, None, None, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), np.repeat(req.numpy()[:, None], k, axis=1))
    rc = np.clip(req.numpy(), 0, R - 1)
    folded = (st.numpy().astype(np.int64) ^ lru.numpy().astype(np.int64))
    # thread t folds slots t, t + 1024, ... (int32 sums) and stores to entries t, t + 1024, ...
    hs.hisparse_diag_floor(None, 2, B, k, S, R, n, d(req), None, d(st), d(lru), None, out)
    torch.cuda.synchronize()
    o2 = out.cpu().numpy().astype(np.int64)
    for b in range(B):
        thread = np.zeros(1024, dtype=np.int64)
        for s in range(S):
            thread[s % 1024] += folded[rc[b], s]
        thread = ((thread + (1 << 31)) % (1 << 32)) - (1 << 31)
        assert np.array_equal(o2[b], thread[np.arange(k) % 1024]), "floor 2, row %d" % b
    hs.hisparse_diag_floor(None, 3, B, k, S, R, n, d(req), d(topk), d(st), d(lru), d(locs), out)
    torch.cuda.synchronize()
    pos = np.clip(topk.numpy().astype(np.int64), 0, n - 1)
    tot = folded[rc].sum(axis=1)                      # the exchange: every slot of the row
    tot = ((tot + (1 << 31)) % (1 << 32)) - (1 << 31)
    pos[tot == -(1 << 31)] = 0                        # as the kernel's address dependence
    want = locs.numpy()[rc[:, None], pos].astype(np.int64) & 0xFFFFFFFF
    want = np.where(want >= 1 << 31, want - (1 << 32), want)
    assert np.array_equal(out.cpu().numpy().astype(np.int64), want), "floor 3"
    full = dict(top_k=k, slots=S, max_requests=R, max_seq_len=n, req_idx=d(req),
                top_k_tokens=d(topk), slot_tokens=d(st), lru_slots=d(lru),
                host_cache_locs=d(locs), out=out)
    for bad in (dict(kind=4, batch=B, **full), dict(kind=0, batch=0),
                dict(kind=1, batch=B, **full, launches=0)):
        try:
            hs.hisparse_diag_floor(None, **bad)
        except hs.HisparseError as e:
            assert e.code == -1
        else:
            raise AssertionError("accepted %s" % bad)
    say("floor kernels compute the stated results; bad kind, batch and launches refused")

    # 4. the last-arriver exchange: sums of every partial, counter left at zero
    xs = torch.zeros((B, hs.EXCHANGE_ROW_INTS), dtype=torch.int32, device=dev)
    for groups in (1, 3, 16):
        hs.hisparse_diag_exchange(None, B, groups, xs, launches=5)
        torch.cuda.synchronize()
        x = xs.cpu().numpy()
        assert (x[:, 0] == 0).all(), "arrival counters not reset"
        want = np.zeros(32, dtype=np.int64)
        for t in range(32):
            want[t] = sum(xx // 64 + xx % 64 for xx in range(t, groups * 64, 256))
        assert (x[:, 32:64] == want[None, :]).all(), ("exchange sums", groups)
    for bad in (dict(batch=B, groups=0), dict(batch=B, groups=17), dict(batch=B, groups=2, launches=0)):
        try:
            hs.hisparse_diag_exchange(None, scratch=xs, **bad)
        except hs.HisparseError as e:
            assert e.code == -1
        else:
            raise AssertionError("accepted %s" % bad)
    say("last-arriver exchange sums every partial and resets its counters")

    # 5. hit detection both ways round: the lowest slot holding each entry's
    #    position (brute force), identical for all four modes; at the largest
    #    shape too (k = S = 4096, where mode 2's table drops to 4 cells per
    #    entry to fit the LDS)
    for B, k, S, R, n in ((6, 900, 700, 4, 5000), (2, 4096, 4096, 2, 20000)):
        req = torch.tensor([0, 3, 1, -2, 7, 2][:B], dtype=torch.int32)
        seq = torch.tensor([5000, 4000, 3000, 5000, 100, 2500][:B], dtype=torch.int32) * (n // 5000)
        topk = torch.stack([torch.randperm(n + 40, generator=g)[:k] - 20 for _ in range(B)]).to(torch.int32)
        st = torch.randint(-3, n, (R, S), generator=g, dtype=torch.int32)
        st[:, 1::7] = st[:, 0::7][:, :st[:, 1::7].shape[1]]   # repeated tokens: the lowest slot wins
        rc = np.clip(req.numpy(), 0, R - 1)
        want = np.full((B, k), -1, dtype=np.int64)
        stn = st.numpy()
        for b in range(B):
            lowest = {}
            for s in range(S - 1, -1, -1):
                lowest[int(stn[rc[b], s])] = s
            for i in range(k):
                t = int(topk[b, i])
                if 0 <= t < min(int(seq[b]), n) and t in lowest:
                    want[b, i] = lowest[t]
        for mode in (0, 1, 2, 3):
            out = torch.full((B, k), -7, dtype=torch.int32, device=dev)
            hs.hisparse_diag_hit_detection(None, mode, B, k, S, R, n, d(req), d(topk), d(seq), d(st), out,
                                           launches=2)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().astype(np.int64), want), ("hit detection", mode, k, S)
        assert (want >= 0).sum() > 100
    say("hit detection both ways round, single-cell and bucketed, gives the lowest slot of every entry's position")
    print("DIAG OK", flush=True)


if __name__ == "__main__":
    main()
