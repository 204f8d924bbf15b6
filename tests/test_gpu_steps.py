"""GPU parity of the multi-step resolver (speculative decoding verification
steps) against consecutive oracle calls, bit-exact, through the C ABI."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from tests.harness import Pair, make_host_pools
from workloads import synth

pytestmark = pytest.mark.gpu


def _mtp_workload(name, seed, B, Q, D, k, L):
    # consecutive synth steps are the Q positions of D decode steps
    # (seq_len + 1 per position), with the pages' hot region (Q + 1) k
    n0 = [3000 + 500 * b for b in range(B)]
    n0[1] = 4 * k - 10          # a request that crosses from the fast path
    return synth(name, seed, R=B + 1, S=(Q + 1) * k, k=k, steps=Q * D, n0=n0, L=L, grow=1,
                 keep=k // 2, recent=k // 4, recent_window=2 * k)


@pytest.mark.parametrize("B", [4, 9])
def test_resolve_steps_vs_oracle(B):
    Q, D, k, L = 4, 5, 64, 2
    print("[steps] B=%d Q=%d" % (B, Q), flush=True)
    w = _mtp_workload("mtp", 50 + B, B, Q, D, k, L)
    bufs = make_host_pools(w)
    pair = Pair(w, bufs, max_steps=Q)
    try:
        out = torch.empty((Q, w.B, w.k), dtype=torch.int32, device="cuda")
        for d in range(D):
            sl = slice(d * Q, (d + 1) * Q)
            for q in range(Q):         # forward-pass writes of fast-path requests
                dst, src = pair.pre_step_writes(d * Q + q)
            hs.hisparse_resolve_steps(pair.pool, None, Q, w.B, w.k, pair.req_idx,
                                      pair.topk[sl].contiguous(), pair.seq[sl].contiguous(),
                                      pair.locs, pair.bt, pair.st, pair.lru, pair.clk, out,
                                      pair.stats)
            o_outs = [pair.oracle_step(d * Q + q, *pair.writes_of(d * Q + q)) for q in range(Q)]
            torch.cuda.synchronize()
            g = out.cpu().numpy()
            for q in range(Q):
                assert np.array_equal(g[q], o_outs[q]), "decode step %d position %d" % (d, q)
            pair.out.copy_(out[Q - 1])
            pair.compare_step(d * Q + Q - 1, o_outs[Q - 1])
            # no position's rows were evicted by a later one: every returned
            # hot row still holds its token, and its bytes are the token's
            st = pair.st.cpu().numpy()
            for q in range(Q):
                tk = w.top_k[d * Q + q]
                for b in range(w.B):
                    r = int(w.req_idx[b])
                    if r < 0:
                        continue
                    for i in np.nonzero(g[q, b] >= 0)[0]:
                        row = int(g[q, b, i])
                        if row < w.R * w.S:
                            assert st[r, row - r * w.S] == tk[b, i]
                rows = np.unique(g[q][g[q] >= 0])
                for l in range(L):
                    dev = pair.dev_pools[l].index_select(
                        0, torch.from_numpy(rows.astype(np.int64)).cuda()).cpu().numpy()
                    assert np.array_equal(dev, pair.ost.dev_pools[l][rows])
            print("[steps] decode step %d ok" % d, flush=True)
        pair.compare_pools()
        # replay of one step's plan restores exactly the rows it copied
        for l in range(L):
            pair.dev_pools[l].zero_()
        hs.hisparse_gather_copy_step(pair.pool, None, 1, w.B)
        torch.cuda.synchronize()
        g1 = out[1].cpu().numpy()
        st = pair.st.cpu().numpy()
        for l in range(L):
            dev = pair.dev_pools[l].cpu().numpy()
            restored = np.nonzero(dev.any(axis=1))[0]
            assert len(restored) > 0
            assert np.array_equal(dev[restored], pair.ost.dev_pools[l][restored])
            assert set(restored.tolist()) <= set(g1[g1 >= 0].tolist())
    finally:
        pair.close()


def test_resolve_steps_bounds():
    w = synth("mtpb", 61, R=4, S=64, k=64, steps=2, n0=[3000, 2000, 900, 5000])
    bufs = make_host_pools(w)
    pair = Pair(w, bufs, max_steps=2)
    try:
        out = torch.empty((3, w.B, w.k), dtype=torch.int32, device="cuda")
        tk = torch.zeros((3, w.B, w.k), dtype=torch.int32, device="cuda")
        sq = torch.ones((3, w.B), dtype=torch.int32, device="cuda")
        with pytest.raises(hs.HisparseError):        # more steps than plan slices
            hs.hisparse_resolve_steps(pair.pool, None, 3, w.B, w.k, pair.req_idx, tk, sq,
                                      pair.locs, pair.bt, pair.st, pair.lru, pair.clk, out)
        with pytest.raises(hs.HisparseError):        # steps * top_k > slots
            hs.hisparse_resolve_steps(pair.pool, None, 2, w.B, w.k, pair.req_idx,
                                      tk[:2].contiguous(), sq[:2].contiguous(), pair.locs, pair.bt,
                                      pair.st, pair.lru, pair.clk, out[:2].contiguous())
        with pytest.raises(hs.HisparseError):        # no such plan slice
            hs.hisparse_gather_copy_step(pair.pool, None, 2, w.B)
        # one step within the bounds is accepted
        hs.hisparse_resolve_steps(pair.pool, None, 1, w.B, w.k, pair.req_idx, pair.topk[:1].contiguous(),
                                  pair.seq[:1].contiguous(), pair.locs, pair.bt, pair.st, pair.lru,
                                  pair.clk, out[:1].contiguous())
        torch.cuda.synchronize()
    finally:
        pair.close()


@pytest.mark.parametrize("seed", range(16))
def test_resolve_steps_random_vs_oracle(seed):
    """Seeded random verification-step calls: 1-4 steps per call, random k,
    batch and layers, hot slots between steps * k and (steps + 2) * k, with or
    without a resident tail (pages of 16 or 24 tokens) and a padding row;
    every position's row IDs, and the state after each call, bit-exact
    against the same positions as consecutive oracle calls."""
    rng = np.random.default_rng(800 + seed)
    Q = int(rng.integers(1, 5))
    D = int(rng.integers(2, 4))
    k = int(rng.integers(1, 97))
    B = int(rng.integers(1, 12))
    L = int(rng.integers(1, 4))
    S = Q * k + int(rng.integers(0, 2 * k + 1))
    n0 = [int(v) for v in rng.integers(1, 8 * S, size=B)]
    keep = int(rng.integers(0, k + 1))
    P = int(rng.choice([0, 0, 16, 24]))
    tail = int(rng.choice([0, 2, 4])) * P
    pad = int(rng.integers(0, 2))
    print("[steps random %d] Q=%d D=%d k=%d S=%d B=%d L=%d P=%d tail=%d pad=%d"
          % (seed, Q, D, k, S, B, L, P, tail, pad), flush=True)
    w = synth("mtprand%d" % seed, 900 + seed, R=B + 1, S=S, k=k, steps=Q * D, n0=n0, L=L, grow=1,
              keep=keep, P=P, resident_tail=tail, padding_rows=pad)
    pair = Pair(w, make_host_pools(w), max_steps=Q)
    try:
        out = torch.empty((Q, w.B, w.k), dtype=torch.int32, device="cuda")
        for d in range(D):
            sl = slice(d * Q, (d + 1) * Q)
            for q in range(Q):
                pair.pre_step_writes(d * Q + q)
            hs.hisparse_resolve_steps(pair.pool, None, Q, w.B, w.k, pair.req_idx,
                                      pair.topk[sl].contiguous(), pair.seq[sl].contiguous(),
                                      pair.locs, pair.bt, pair.st, pair.lru, pair.clk, out,
                                      pair.stats)
            o_outs = [pair.oracle_step(d * Q + q, *pair.writes_of(d * Q + q)) for q in range(Q)]
            torch.cuda.synchronize()
            g = out.cpu().numpy()
            for q in range(Q):
                assert np.array_equal(g[q], o_outs[q]), "decode step %d position %d" % (d, q)
            pair.out.copy_(out[Q - 1])
            pair.compare_step(d * Q + Q - 1, o_outs[Q - 1])
        pair.compare_pools()
    finally:
        pair.close()
