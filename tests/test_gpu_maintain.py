"""GPU parity of the row mirror and of hot-entry invalidation against the
CPU oracle (bit-exact), through the C ABI."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from oracle import (OracleState, oracle_invalidate_host_rows, oracle_invalidate_tokens,
                    oracle_mirror_rows, oracle_resolve)
from tests.harness import Pair, make_host_pools
from workloads import synth

pytestmark = pytest.mark.gpu
RB = 656


def _small_pool(R, S, L, dev_rows, host_rows, max_seq_len=64, rb=RB):
    bufs = [hs.HostBuffer(host_rows * rb) for _ in range(L)]
    for l, hb in enumerate(bufs):
        hb.numpy((host_rows, rb))[:] = 0x5A + l
    devs = [torch.randint(0, 256, (dev_rows, rb), dtype=torch.uint8, device="cuda",
                          generator=torch.Generator(device="cuda").manual_seed(7 + l))
            for l in range(L)]
    cfg = hs.PoolConfig(max_requests=R, slots=S, max_top_k=min(S, 64), max_batch=8, row_bytes=rb,
                        num_layers=L, max_seq_len=max_seq_len)
    pool = hs.hisparse_init_pool(cfg, bufs, [host_rows] * L, devs, dev_rows)
    return pool, bufs, devs


@pytest.mark.parametrize("count,rb", [(1, RB), (37, RB), (5000, RB), (37, 16), (600, 2064)])
def test_mirror_rows_vs_oracle(count, rb):
    """Rows of 656 bytes, of one 16-byte unit, and of 129 units (more than one
    per lane)."""
    print("[mirror] count=%d row_bytes=%d" % (count, rb), flush=True)
    L, dev_rows, host_rows = 2, 6000, 9000
    pool, bufs, devs = _small_pool(R=4, S=1024, L=L, dev_rows=dev_rows, host_rows=host_rows, rb=rb)
    try:
        rng = np.random.default_rng(count)
        d = rng.integers(0, dev_rows, size=count).astype(np.int32)
        h = rng.choice(host_rows, size=count, replace=False).astype(np.int64)
        if count > 3:
            d[1] = -1                      # padding
            d[2] = dev_rows + 3            # past the device pool: tripwire
            h[3] = host_rows               # past the host pool: tripwire
        ost = OracleState(R=4, S=1024, L=L, row_bytes=rb, dev_pool_rows=dev_rows)
        for l in range(L):
            ost.dev_pools[l][:] = devs[l].cpu().numpy()
        ohost = [b.numpy((host_rows, rb)).copy() for b in bufs]
        oracle_mirror_rows(ost, dev_rows=d, host_rows=h, host_pools=ohost,
                           host_pool_rows=[host_rows] * L, validate=True)
        stats = torch.zeros(5, dtype=torch.int64, device="cuda")
        hs.hisparse_mirror_rows(pool, None, torch.from_numpy(d).cuda(), torch.from_numpy(h).cuda(),
                                stats=stats)
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(bufs[l].numpy((host_rows, rb)), ohost[l]), "layer %d" % l
        assert np.array_equal(stats.cpu().numpy().astype(np.uint64), ost.stats)
        # a layer range touches only its layers
        hs.hisparse_mirror_rows(pool, None, torch.from_numpy(d[:1].copy()).cuda(),
                                torch.from_numpy(np.array([0], np.int64)).cuda(), 1, 2)
        torch.cuda.synchronize()
        assert np.array_equal(bufs[0].numpy((host_rows, rb))[0], ohost[0][0])
        if d[0] >= 0:
            assert np.array_equal(bufs[1].numpy((host_rows, rb))[0], ost.dev_pools[1][d[0]])
    finally:
        hs.hisparse_destroy_pool(pool)
        for b in bufs:
            b.free()


@pytest.mark.parametrize("mode", ["resolve", "split"])
def test_live_decode_loop_with_mirror(mode):
    """The forward pass writes each new token's row on the device (hot row
    on the fast path, a staging row otherwise); the mirror copies it to its
    host row, whose old bytes were cleared; later steps select those tokens
    and must fetch exactly the written bytes.  GPU and oracle run the same
    sequence; every step is compared."""
    print("[live loop %s]" % mode, flush=True)
    w = synth("live", 41, R=10, S=256, k=96, steps=12,
              n0=[2000, 250, 254, 3000, 900, 128, 5000, 4000, 700], L=2, grow=1, keep=60,
              recent=20, recent_window=24, padding_rows=1)
    staging0 = w.dev_pool_rows
    w.extra_dev_rows = w.B
    bufs = make_host_pools(w)
    # host rows of the tokens appended during the run hold no data yet
    new_rows = []
    for b in range(w.B):
        r = int(w.req_idx[b])
        if r >= 0:
            new_rows.extend(w.host_cache_locs[r, int(w.seq_lens[0, b]):int(w.seq_lens[-1, b])].tolist())
    for hb in bufs:
        hb.numpy((w.host_pool_rows, RB))[new_rows] = 0
    pair = Pair(w, bufs, mode=mode)
    ohost = [a.copy() for a in pair.host_np]
    rng = np.random.default_rng(5)
    stats_m = torch.zeros(5, dtype=torch.int64, device="cuda")
    try:
        for step in range(w.steps):
            if step > 0:
                d, h, rows = [], [], []
                for b in range(w.B):
                    r = int(w.req_idx[b])
                    if r < 0:
                        continue
                    for t in range(int(w.seq_lens[step - 1, b]), int(w.seq_lens[step, b])):
                        dev_row = r * w.S + t if w.seq_lens[step, b] <= w.S else staging0 + b
                        d.append(dev_row)
                        h.append(int(w.host_cache_locs[r, t]))
                d = np.array(d, np.int32)
                h = np.array(h, np.int64)
                for l in range(w.L):
                    content = rng.integers(0, 256, size=(len(d), RB), dtype=np.uint8)
                    pair.dev_pools[l][torch.from_numpy(d.astype(np.int64)).cuda()] = \
                        torch.from_numpy(content).cuda()
                    pair.ost.dev_pools[l][d] = content
                hs.hisparse_mirror_rows(pair.pool, None, torch.from_numpy(d).cuda(),
                                        torch.from_numpy(h).cuda(), stats=stats_m)
                oracle_mirror_rows(pair.ost, dev_rows=d, host_rows=h, host_pools=ohost,
                                   host_pool_rows=[w.host_pool_rows] * w.L, validate=True)
            args = (pair.pool, None, w.B, w.k, pair.req_idx, pair.topk[step], pair.seq[step],
                    pair.locs, pair.bt, pair.st, pair.lru, pair.clk, pair.out, pair.stats)
            if mode == "resolve":
                hs.hisparse_resolve(*args)
            else:
                hs.hisparse_resolve_plan(*args)
                hs.hisparse_gather_copy(pair.pool, None, w.B, 0, w.L, pair.stats)
            o_out = oracle_resolve(pair.ost, page_size=w.P, max_seq_len=w.max_seq_len,
                                   resident_pages=w.resident_pages, req_idx=w.req_idx,
                                   top_k_tokens=w.top_k[step], seq_lens=w.seq_lens[step],
                                   host_cache_locs=w.host_cache_locs, block_table=w.block_table,
                                   host_pools=ohost, host_pool_rows=[w.host_pool_rows] * w.L)
            torch.cuda.synchronize()
            pair.compare_step(step, o_out)
        for l in range(w.L):
            assert np.array_equal(pair.host_np[l], ohost[l])
        assert int(stats_m[4]) == 0
        # the run did select tokens that only the mirror had put on the host
        sel = set()
        for step in range(1, w.steps):
            for b in range(w.B):
                r = int(w.req_idx[b])
                if r >= 0:
                    sel.update(int(w.host_cache_locs[r, t]) for t in w.top_k[step, b] if t >= 0)
        assert sel & set(new_rows)
    finally:
        pair.close()


def _random_state(rng, R, S, n):
    st = np.full((R, S), -1, np.int32)
    lru = np.zeros((R, S), np.int32)
    for r in range(R):
        occ = rng.random(S) < 0.85
        st[r] = np.where(occ, rng.permutation(n)[:S], -1)
        lru[r] = np.where(occ, rng.integers(1, 1 << 20, S), 0)
    st[0, :4] = [-5, n + 10, -1, 3]
    return st, lru


@pytest.mark.parametrize("R,S,n,nset", [(6, 300, 1000, 50), (72, 4096, 131072, 5000),
                                        (72, 4096, 131072, 20000)])
def test_invalidate_host_rows_vs_oracle(R, S, n, nset):
    print("[invalidate rows] R=%d S=%d set=%d" % (R, S, nset), flush=True)
    rng = np.random.default_rng(nset)
    st, lru = _random_state(rng, R, S, n)
    locs = rng.integers(0, R * n, size=(R, n)).astype(np.int64)
    rows = np.sort(rng.choice(R * n, size=nset, replace=False)).astype(np.int64)
    hb = hs.HostBuffer(RB * 16)
    dev = torch.zeros((R * S, RB), dtype=torch.uint8, device="cuda")
    cfg = hs.PoolConfig(max_requests=R, slots=S, max_top_k=min(S, 64), max_batch=1, row_bytes=RB,
                        max_seq_len=n)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], R * S)
    try:
        gst, glru = torch.from_numpy(st).cuda(), torch.from_numpy(lru).cuda()
        hs.hisparse_invalidate_host_rows(pool, None, torch.from_numpy(rows).cuda(),
                                         torch.from_numpy(locs).cuda(), gst, glru)
        ost = OracleState(R=R, S=S, L=1, row_bytes=RB, dev_pool_rows=1)
        ost.slot_tokens[:], ost.lru_slots[:] = st, lru
        oracle_invalidate_host_rows(ost, rows=rows, host_cache_locs=locs, max_seq_len=n,
                                    validate=True)
        torch.cuda.synchronize()
        assert np.array_equal(gst.cpu().numpy(), ost.slot_tokens)
        assert np.array_equal(glru.cpu().numpy(), ost.lru_slots)
        assert (ost.slot_tokens != st).sum() > 0
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


@pytest.mark.parametrize("R,S", [(5, 77), (72, 4096)])
def test_invalidate_tokens_vs_oracle(R, S):
    print("[invalidate tokens] R=%d S=%d" % (R, S), flush=True)
    rng = np.random.default_rng(S)
    n = 50000
    st, lru = _random_state(rng, R, S, n)
    cnt = 40
    req = rng.integers(0, R, cnt).astype(np.int32)
    req[0], req[1] = -1, R + 3                  # padding, out of range (tripwire)
    b = rng.integers(0, n, cnt).astype(np.int32)
    e = (b + rng.integers(0, 3000, cnt)).astype(np.int32)
    b[2], e[2] = 0, 2 ** 31 - 1                 # a whole request row
    hb = hs.HostBuffer(RB * 16)
    dev = torch.zeros((R * S, RB), dtype=torch.uint8, device="cuda")
    cfg = hs.PoolConfig(max_requests=R, slots=S, max_top_k=min(S, 64), max_batch=1, row_bytes=RB,
                        max_seq_len=16)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], R * S)
    try:
        gst, glru = torch.from_numpy(st).cuda(), torch.from_numpy(lru).cuda()
        stats = torch.zeros(5, dtype=torch.int64, device="cuda")
        hs.hisparse_invalidate_tokens(pool, None, torch.from_numpy(req).cuda(),
                                      torch.from_numpy(b).cuda(), torch.from_numpy(e).cuda(),
                                      gst, glru, stats)
        ost = OracleState(R=R, S=S, L=1, row_bytes=RB, dev_pool_rows=1)
        ost.slot_tokens[:], ost.lru_slots[:] = st, lru
        oracle_invalidate_tokens(ost, req_rows=req, tok_begin=b, tok_end=e)
        torch.cuda.synchronize()
        assert np.array_equal(gst.cpu().numpy(), ost.slot_tokens)
        assert np.array_equal(glru.cpu().numpy(), ost.lru_slots)
        assert np.array_equal(stats.cpu().numpy().astype(np.uint64), ost.stats)
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


def test_invalidate_then_resolve_refetches():
    """Host rows of some cached tokens are rewritten and invalidated; the next
    resolver step misses on exactly those and copies the new bytes."""
    print("[invalidate + resolve]", flush=True)
    w = synth("inv", 43, R=4, S=256, k=128, steps=2, n0=[3000, 2500, 4000, 6000], keep=128)
    bufs = make_host_pools(w)
    pair = Pair(w, bufs)
    try:
        dst, src = pair.gpu_step(0)
        o = pair.oracle_step(0, dst, src)
        torch.cuda.synchronize()
        pair.compare_step(0, o)
        rng = np.random.default_rng(1)
        cached = np.unique(w.host_cache_locs[w.req_idx[0], w.top_k[0, 0][w.top_k[0, 0] >= 0]])
        rows = np.sort(rng.choice(cached, size=20, replace=False)).astype(np.int64)
        pair.host_np[0][rows] = 0xC3               # the oracle reads the same host memory
        hs.hisparse_invalidate_host_rows(pair.pool, None, torch.from_numpy(rows).cuda(), pair.locs,
                                         pair.st, pair.lru)
        oracle_invalidate_host_rows(pair.ost, rows=rows, host_cache_locs=w.host_cache_locs,
                                    max_seq_len=w.max_seq_len, validate=True)
        before = pair.ost.stats.copy()
        dst, src = pair.gpu_step(1)
        o = pair.oracle_step(1, dst, src)
        torch.cuda.synchronize()
        pair.compare_step(1, o)
        assert pair.ost.stats[1] - before[1] >= 20
    finally:
        pair.close()


def test_empty_calls_change_nothing():
    """Zero entries: the mirror, both invalidations and an empty layer range
    return without touching host pools, device pools or state."""
    R, S, n, L = 4, 256, 600, 2
    pool, bufs, devs = _small_pool(R=R, S=S, L=L, dev_rows=R * S, host_rows=700, max_seq_len=n)
    try:
        rng = np.random.default_rng(3)
        st, lru = _random_state(rng, R, S, n)
        gst, glru = torch.from_numpy(st).cuda(), torch.from_numpy(lru).cuda()
        locs = torch.from_numpy(rng.integers(0, 700, size=(R, n)).astype(np.int64)).cuda()
        host0 = [b.numpy((700, RB)).copy() for b in bufs]
        dev0 = [d.clone() for d in devs]
        stats = torch.zeros(5, dtype=torch.int64, device="cuda")
        e32 = torch.empty(0, dtype=torch.int32, device="cuda")
        e64 = torch.empty(0, dtype=torch.int64, device="cuda")
        hs.hisparse_mirror_rows(pool, None, e32, e64, stats=stats)
        one = torch.zeros(1, dtype=torch.int32, device="cuda")
        hs.hisparse_mirror_rows(pool, None, one, torch.zeros(1, dtype=torch.int64, device="cuda"),
                                1, 1, stats=stats)  # an empty layer range
        hs.hisparse_invalidate_tokens(pool, None, e32, e32, e32, gst, glru, stats)
        hs.hisparse_invalidate_host_rows(pool, None, e64, locs, gst, glru)
        torch.cuda.synchronize()
        for l in range(L):
            assert np.array_equal(bufs[l].numpy((700, RB)), host0[l])
            assert torch.equal(devs[l], dev0[l])
        assert np.array_equal(gst.cpu().numpy(), st) and np.array_equal(glru.cpu().numpy(), lru)
        assert int(stats.sum().item()) == 0
    finally:
        hs.hisparse_destroy_pool(pool)
        for b in bufs:
            b.free()
