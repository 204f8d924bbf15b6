"""Pins of the CPU oracle against facts fixed outside of it (CPU only).

Each test ties the oracle to something it does not share code with:
hand-worked cases, the textbook LRU cache, set counts, an independent
formulation on exhaustive tiny inputs, step invariants, the OCP fp8 and
bfloat16 definitions via torch's CPU codecs, and torch's float64 attention.
"""
import itertools
import math
import os
from collections import OrderedDict

import numpy as np
import pytest
import torch

from oracle import (OracleState, bf16_to_double, e4m3_to_double, oracle_resolve,
                    oracle_sparse_mla_decode)
from tests.naive_resolver import naive_resolve

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RB = 16  # row bytes for tiny resolver tests


def _host_pool(rows, layers=1, row_bytes=RB, seed=0):
    rng = np.random.default_rng(seed)
    return [rng.integers(0, 256, size=(rows, row_bytes), dtype=np.uint8) for _ in range(layers)]


# ---------------------------------------------------------------- codecs --

def test_e4m3_spec_points():
    for line in open(os.path.join(GOLDEN, "e4m3_spec_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = e4m3_to_double(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_exhaustive_vs_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = e4m3_to_double(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])


def test_bf16_exhaustive_vs_torch():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    for v in range(0, 65536, 7):
        got = bf16_to_double(v)
        if math.isnan(ref[v]):
            assert math.isnan(got)
        else:
            assert got == ref[v]


# ---------------------------------------------------- resolver: by hand --

def test_worked_example():
    R, S, P = 2, 4, 4
    st = OracleState(R=R, S=S, L=1, row_bytes=RB, dev_pool_rows=R * S + 1 * P)
    st.slot_tokens[1] = [5, -1, 7, 9]
    st.lru_slots[1] = [3, 0, 1, 1]
    st.lru_clock[1] = 3
    locs = np.full((R, 16), -1, np.int64)
    locs[1] = 100 + np.arange(16)
    bt = np.full((R, 4), -1, np.int32)
    bt[1, 3] = 0
    host = _host_pool(200)
    for line in open(os.path.join(GOLDEN, "resolver_worked_example.txt")):
        if not line.startswith("call"):
            continue
        f = [x.split() for x in line.split("|")]
        topk = np.array([[int(x) for x in f[0][3:]]], np.int32)
        out = oracle_resolve(st, page_size=P, max_seq_len=16, resident_pages=1,
                             req_idx=[1], top_k_tokens=topk, seq_lens=[16],
                             host_cache_locs=locs, block_table=bt, host_pools=host,
                             host_pool_rows=[200], validate=True)
        assert out[0].tolist() == [int(x) for x in f[1][1:]]
        assert st.slot_tokens[1].tolist() == [int(x) for x in f[2][1:]]
        assert st.lru_slots[1].tolist() == [int(x) for x in f[3][1:]]
        assert int(st.lru_clock[1]) == int(f[4][1])
        assert st.stats.tolist() == [int(x) for x in f[5][1:]]
    # copied bytes: the slots filled by misses hold their token's host row
    # (slot 3 kept token 9 from the initial state and was never copied)
    for s in range(3):
        t = st.slot_tokens[1, s]
        assert np.array_equal(st.dev_pools[0][1 * S + s], host[0][100 + t])


# --------------------------------------------- resolver: textbook LRU --

@pytest.mark.parametrize("S,n,seed", [(1, 5, 0), (3, 10, 1), (5, 12, 2), (8, 40, 3)])
def test_k1_is_textbook_lru(S, n, seed):
    """With top-k = 1 the resolver is an LRU cache of S entries: free slots
    are filled lowest first, then the least recently used entry is evicted."""
    rng = np.random.default_rng(seed)
    st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
    locs = np.arange(n, dtype=np.int64)[None, :]
    host = _host_pool(n)
    cache = OrderedDict()      # token -> slot, least recent first
    free = list(range(S))
    hits = misses = 0
    for step in range(300):
        t = int(rng.integers(-1, n)) if step % 17 else -1
        out = oracle_resolve(st, page_size=0, max_seq_len=n, resident_pages=0,
                             req_idx=[0], top_k_tokens=[[t]], seq_lens=[n],
                             host_cache_locs=locs, block_table=None, host_pools=host,
                             host_pool_rows=[n])
        if t < 0:
            assert out[0, 0] == -1
            continue
        if t in cache:
            cache.move_to_end(t)
            hits += 1
        else:
            slot = free.pop(0) if free else cache.popitem(last=False)[1]
            cache[t] = slot
            misses += 1
        assert out[0, 0] == cache[t]
    assert st.stats[0] == hits and st.stats[1] == misses
    assert sorted(cache.items()) == sorted((int(st.slot_tokens[0, s]), s)
                                           for s in range(S) if st.slot_tokens[0, s] >= 0)


# ------------------------------------------------ resolver: set counts --

def test_big_buffer_misses_are_first_occurrences():
    """When the buffer holds every position ever asked for, misses equal the
    number of distinct positions and every repeat is a hit."""
    rng = np.random.default_rng(7)
    S, k, n, steps = 64, 8, 100, 40
    universe = rng.choice(n, size=60, replace=False)
    st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
    locs = np.arange(n, dtype=np.int64)[None, :]
    host = _host_pool(n)
    seen, total = set(), 0
    for _ in range(steps):
        row = rng.choice(universe, size=k, replace=False).astype(np.int32)
        oracle_resolve(st, page_size=0, max_seq_len=n, resident_pages=0, req_idx=[0],
                       top_k_tokens=row[None], seq_lens=[n], host_cache_locs=locs,
                       block_table=None, host_pools=host, host_pool_rows=[n])
        seen.update(row.tolist())
        total += k
    assert st.stats[1] == len(seen)
    assert st.stats[0] == total - len(seen)


def test_full_reuse_has_no_misses_after_step0():
    rng = np.random.default_rng(8)
    S, k, n = 32, 16, 200
    base = rng.choice(n, size=k, replace=False).astype(np.int32)
    st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
    locs = np.arange(n, dtype=np.int64)[None, :]
    host = _host_pool(n)
    for step in range(10):
        row = rng.permutation(base)
        oracle_resolve(st, page_size=0, max_seq_len=n, resident_pages=0, req_idx=[0],
                       top_k_tokens=row[None], seq_lens=[n], host_cache_locs=locs,
                       block_table=None, host_pools=host, host_pool_rows=[n])
        assert st.stats[1] == k          # all misses happened at step 0
        assert st.stats[0] == k * step


def test_cold_step_gives_jth_miss_slot_j():
    rng = np.random.default_rng(9)
    R, S, k, n = 3, 64, 40, 500
    st = OracleState(R=R, S=S, L=1, row_bytes=RB, dev_pool_rows=R * S)
    locs = np.arange(R * n, dtype=np.int64).reshape(R, n)
    host = _host_pool(R * n)
    topk = np.stack([rng.choice(n, size=k, replace=False) for _ in range(R)]).astype(np.int32)
    topk[1, ::5] = -1
    out = oracle_resolve(st, page_size=0, max_seq_len=n, resident_pages=0,
                         req_idx=[2, 0, 1], top_k_tokens=topk, seq_lens=[n] * R,
                         host_cache_locs=locs, block_table=None, host_pools=host,
                         host_pool_rows=[R * n])
    for b, r in enumerate([2, 0, 1]):
        j = 0
        for i in range(k):
            if topk[b, i] < 0:
                assert out[b, i] == -1
            else:
                assert out[b, i] == r * S + j
                j += 1


# ---------------------------------- resolver: independent formulation --

def _run_both(R, S, P, n, steps_topk, *, seq=None, bt=None, resident_pages=0,
              init=None, req_idx=None, locs=None, host_rows=None, L=1):
    """Run the oracle and the naive formulation side by side; compare all."""
    B = steps_topk[0].shape[0]
    req_idx = np.arange(B, dtype=np.int32) if req_idx is None else np.asarray(req_idx, np.int32)
    seq = np.full(B, n, np.int32) if seq is None else np.asarray(seq, np.int32)
    if locs is None:
        locs = np.arange(R * n, dtype=np.int64).reshape(R, n)
    host_rows = [R * n] * L if host_rows is None else host_rows
    host = _host_pool(max(host_rows) + 1, layers=L, seed=5)
    dev_rows = R * S + resident_pages * max(P, 0)
    ost = OracleState(R=R, S=S, L=L, row_bytes=RB, dev_pool_rows=dev_rows)
    if init is not None:
        ost.slot_tokens[:], ost.lru_slots[:], ost.lru_clock[:] = init
    n_st, n_lru, n_clk = ost.slot_tokens.copy(), ost.lru_slots.copy(), ost.lru_clock.copy()
    n_stats = np.zeros(5, np.uint64)
    n_pools = [p.copy() for p in ost.dev_pools]
    for topk in steps_topk:
        o1 = oracle_resolve(ost, page_size=P, max_seq_len=n, resident_pages=resident_pages,
                            req_idx=req_idx, top_k_tokens=topk, seq_lens=seq,
                            host_cache_locs=locs, block_table=bt, host_pools=host,
                            host_pool_rows=host_rows)
        o2 = naive_resolve(n_st, n_lru, n_clk, n_stats, n_pools, R=R, S=S, P=P,
                           max_seq_len=n, resident_pages=resident_pages, req_idx=req_idx,
                           topk=np.asarray(topk), seq_lens=seq, locs=locs, bt=bt,
                           host_pools=host, host_rows=host_rows, row_bytes=RB)
        assert np.array_equal(o1, o2)
        assert np.array_equal(ost.slot_tokens, n_st)
        assert np.array_equal(ost.lru_slots, n_lru)
        assert np.array_equal(ost.lru_clock, n_clk)
        assert np.array_equal(ost.stats, n_stats)
        for a, b in zip(ost.dev_pools, n_pools):
            assert np.array_equal(a, b)


def _ordered_rows(k, n):
    """All top-k rows over {-1, 0..n-1} with distinct valid entries."""
    rows = []
    for tup in itertools.product(range(-1, n), repeat=k):
        v = [t for t in tup if t >= 0]
        if len(v) == len(set(v)):
            rows.append(tup)
    return rows


@pytest.mark.parametrize("S,k,n", [(1, 1, 3), (2, 1, 4), (2, 2, 4), (3, 2, 5), (3, 3, 5), (4, 3, 6)])
def test_exhaustive_two_steps_vs_naive(S, k, n):
    """Every pair of consecutive top-k rows on a tiny request, each pair its
    own request row, all in one call per step."""
    rows = _ordered_rows(k, n)
    pairs = list(itertools.product(rows, repeat=2))
    if len(pairs) > 6000:
        rng = np.random.default_rng(S * 100 + k * 10 + n)
        pairs = [pairs[i] for i in rng.choice(len(pairs), 6000, replace=False)]
    B = len(pairs)
    steps = [np.array([p[s] for p in pairs], np.int32) for s in range(2)]
    _run_both(B, S, 0, n, steps)


@pytest.mark.parametrize("S,k,n", [(2, 1, 4), (2, 2, 3), (3, 2, 4)])
def test_exhaustive_three_steps_vs_naive(S, k, n):
    rows = _ordered_rows(k, n)
    triples = list(itertools.product(rows, repeat=3))
    if len(triples) > 8000:
        rng = np.random.default_rng(S * 100 + k * 10 + n + 1)
        triples = [triples[i] for i in rng.choice(len(triples), 8000, replace=False)]
    B = len(triples)
    steps = [np.array([p[s] for p in triples], np.int32) for s in range(3)]
    _run_both(B, S, 0, n, steps)


@pytest.mark.parametrize("P", [4, 3, 5])
@pytest.mark.parametrize("seed", range(6))
def test_random_corrupt_state_vs_naive(seed, P):
    """Random initial state including empty markers below -1, one position in
    two slots, stamps above the clock and negative stamps, with a resident
    block table (some entries out of range; pages of 3, 4 or 5 tokens, the
    last page partial for 3), padding rows, request indices past R,
    out-of-range host rows and invalid top-k entries."""
    rng = np.random.default_rng(100 + seed + 1000 * (P != 4) * P)
    R, S, n, k, L = 6, 8, 40, 6, 2
    st0 = rng.integers(-3, n + 3, size=(R, S)).astype(np.int32)
    st0[0, 1] = st0[0, 5] = 11          # one position held twice
    lru0 = rng.integers(-2, 6, size=(R, S)).astype(np.int32)
    clk0 = rng.integers(0, 4, size=R).astype(np.int32)
    resident_pages = 3
    bt = rng.integers(-1, resident_pages + 2, size=(R, -(-n // P))).astype(np.int32)
    bt[bt < 1] = -1
    bt[bt >= 1] -= 1                    # some >= resident_pages (corrupt)
    locs = rng.integers(-2, R * n + 5, size=(R, n)).astype(np.int64)
    req_idx = np.array([3, -1, 0, R + 1, 5, 1], np.int32)
    seq = np.array([n, n, n - 7, n, n + 10, 9], np.int32)   # row 5: fast path
    steps = []
    for _ in range(5):
        rows = []
        for b in range(len(req_idx)):
            row = rng.choice(np.arange(-1, n + 4), size=k, replace=False)
            rows.append(row)
        steps.append(np.array(rows, np.int32))
    _run_both(R, S, P, n, steps, seq=seq, bt=bt, resident_pages=resident_pages,
              init=(st0, lru0, clk0), req_idx=req_idx, locs=locs,
              host_rows=[R * n, R * n - 30], L=L)


def test_oracle_rejects_duplicates_when_validating():
    st = OracleState(R=2, S=4, L=1, row_bytes=RB, dev_pool_rows=8)
    locs = np.arange(40, dtype=np.int64).reshape(2, 20)
    host = _host_pool(40)
    with pytest.raises(ValueError):
        oracle_resolve(st, page_size=0, max_seq_len=20, resident_pages=0, req_idx=[0],
                       top_k_tokens=[[3, 4, 3]], seq_lens=[20], host_cache_locs=locs,
                       block_table=None, host_pools=host, host_pool_rows=[40], validate=True)
    with pytest.raises(ValueError):
        oracle_resolve(st, page_size=0, max_seq_len=20, resident_pages=0, req_idx=[1, 1],
                       top_k_tokens=[[3], [4]], seq_lens=[20, 20], host_cache_locs=locs,
                       block_table=None, host_pools=host, host_pool_rows=[40], validate=True)
    assert st.lru_clock.tolist() == [0, 0]


# ---------------------------------------------- resolver: invariants --

def check_step_invariants(w, step, before, after, out, host_pools, dev_pools, c_expected):
    """Invariants of one resolver step on a workload (no corruption)."""
    (st0, lru0), (st1, lru1) = before, after
    S = w.S
    topk, seq = w.top_k[step], w.seq_lens[step]
    for b in range(w.B):
        r = int(w.req_idx[b])
        if r < 0:
            assert (out[b] == -1).all()
            continue
        n = int(seq[b])
        c = c_expected[r]
        valid = (topk[b] >= 0) & (topk[b] < n)
        assert (out[b][~valid] == -1).all()
        assert (out[b][valid] >= 0).all()                 # every position resolved
        hot = valid & (out[b] < w.R * S)
        slots = out[b][hot] - r * S
        assert ((slots >= 0) & (slots < S)).all()
        assert len(np.unique(slots)) == len(slots)        # distinct slots
        assert (st1[r, slots] == topk[b][hot]).all()      # slot holds its token
        assert (lru1[r, slots] == c).all()                # touched stamps == c
        if n <= S:
            assert (out[b][valid] == r * S + topk[b][valid]).all()   # identity
            continue
        occ = st1[r][st1[r] >= 0]
        assert len(np.unique(occ)) == len(occ)            # no position twice
        hit_mask = np.zeros(S, bool)
        for s in slots:
            if st0[r, s] == st1[r, s]:
                hit_mask[s] = True                         # kept token: a hit
        changed = np.nonzero(st0[r] != st1[r])[0]
        # every victim's key is below every unchosen non-hit slot's key
        key = lambda s: (1 if st0[r, s] >= 0 else 0, int(lru0[r, s]), int(s))
        untouched = [s for s in range(S) if not hit_mask[s] and s not in set(changed)
                     and not (lru1[r, s] == c and st0[r, s] == st1[r, s])]
        if len(changed) and untouched:
            assert max(key(s) for s in changed) < min(key(s) for s in untouched)
        # global content invariant
        for s in range(S):
            t = st1[r, s]
            if t >= 0:
                h = w.host_cache_locs[r, t]
                for l in range(w.L):
                    assert np.array_equal(dev_pools[l][r * S + s], host_pools[l][h])


@pytest.mark.parametrize("row_bytes,L", [(656, 1), (16, 2), (2064, 2)])
def test_step_invariants_on_small_workload(row_bytes, L):
    """Every step's invariants, including every hot row's bytes against its
    token's host row in every layer, at row widths of one 16-byte unit up to
    129 units."""
    from workloads import synth, admission, decode_writes, fill_host_rows_uniform
    w = synth("small", 11, R=6, S=64, k=24, steps=12, n0=[300, 500, 40, 64, 1000, 62],
              grow=1, keep=20, recent=2, recent_window=30, padding_rows=1, L=L)
    w.row_bytes = row_bytes
    hostt = [torch.empty((w.host_pool_rows, row_bytes), dtype=torch.uint8) for _ in range(w.L)]
    for l, h in enumerate(hostt):
        fill_host_rows_uniform(h, seed=50 + l)
    host = [h.numpy() for h in hostt]
    st = OracleState(R=w.R, S=w.S, L=w.L, row_bytes=row_bytes, dev_pool_rows=w.dev_pool_rows)
    s0, l0, c0, dst, src = admission(w)
    st.slot_tokens[:], st.lru_slots[:], st.lru_clock[:] = s0, l0, c0
    for l in range(w.L):
        st.dev_pools[l][dst] = host[l][src]
    for step in range(w.steps):
        d, s = decode_writes(w, step)
        for l in range(w.L):
            st.dev_pools[l][d] = host[l][s]
        before = (st.slot_tokens.copy(), st.lru_slots.copy())
        c_exp = st.lru_clock.copy() + 1
        out = oracle_resolve(st, page_size=0, max_seq_len=w.max_seq_len, resident_pages=0,
                             req_idx=w.req_idx, top_k_tokens=w.top_k[step],
                             seq_lens=w.seq_lens[step], host_cache_locs=w.host_cache_locs,
                             block_table=None, host_pools=host,
                             host_pool_rows=[w.host_pool_rows] * w.L, validate=True)
        check_step_invariants(w, step, before, (st.slot_tokens, st.lru_slots), out, host,
                              st.dev_pools, c_exp)
    assert st.stats[4] == 0


# -------------------------------------------------- attention pins --

def _mla_rows(m, seed):
    from workloads import fill_host_rows_mla
    t = torch.empty((m, 656), dtype=torch.uint8)
    fill_host_rows_mla(t, seed)
    return t


def _torch_reference(q_bits, locs, pool, scale):
    """float64 attention with torch's own fp8/bf16 decoders and softmax."""
    B, H, _ = q_bits.shape
    q = torch.from_numpy(q_bits.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    out = torch.zeros((B, H, 512), dtype=torch.float64)
    for b in range(B):
        sel = [int(x) for x in locs[b] if 0 <= x < pool.shape[0]]
        if not sel:
            continue
        rows = pool[sel]
        lat = rows[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
        sc = rows[:, 512:528].contiguous().view(torch.float32).to(torch.float64)
        deq = (lat.reshape(-1, 4, 128) * sc[:, :, None]).reshape(-1, 512)
        rope = rows[:, 528:656].contiguous().view(torch.bfloat16).to(torch.float64)
        K = torch.cat([deq, rope], dim=1)
        z = (q[b] @ K.T) * scale
        out[b] = torch.softmax(z, dim=1) @ deq
    return out.numpy()


def test_attention_vs_torch_float64():
    pool = _mla_rows(300, seed=3)
    rng = np.random.default_rng(4)
    B, H, k = 3, 8, 37
    locs = np.stack([rng.choice(300, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    locs[1, ::3] = -1
    locs[2, :] = -1
    locs[2, 5] = 17
    q = torch.randn((B, H, 576), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().astype(np.uint16)
    scale = float(np.float32(1.0 / math.sqrt(192.0)))
    got = oracle_sparse_mla_decode(q_bits, locs, pool.numpy(), scale)
    ref = _torch_reference(q_bits, locs, pool, scale)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("row_bytes", [672, 1024])
def test_attention_padded_rows_vs_torch_float64(row_bytes):
    """Rows stored at a larger stride: the oracle reads each row's 656-byte
    record at that stride and never the padding (all 0xFF, NaN codes), so it
    equals torch's float64 attention over the unpadded rows."""
    pool = _mla_rows(200, seed=8)
    padded = torch.full((200, row_bytes), 0xFF, dtype=torch.uint8)
    padded[:, :656] = pool
    rng = np.random.default_rng(row_bytes)
    B, H, k = 2, 8, 29
    locs = np.stack([rng.choice(200, size=k, replace=False) for _ in range(B)]).astype(np.int32)
    locs[0, ::4] = -1
    q = torch.randn((B, H, 576), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().astype(np.uint16)
    scale = float(np.float32(1.0 / math.sqrt(192.0)))
    got = oracle_sparse_mla_decode(q_bits, locs, padded.numpy(), scale, row_bytes=row_bytes)
    ref = _torch_reference(q_bits, locs, pool, scale)
    assert np.isfinite(got).all()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    pool = _mla_rows(64, seed=6)
    H = 4
    scale = float(np.float32(1.0 / math.sqrt(192.0)))
    deq = (pool[:, :512].contiguous().view(torch.float8_e4m3fn).to(torch.float64).reshape(-1, 4, 128)
           * pool[:, 512:528].contiguous().view(torch.float32).to(torch.float64)[:, :, None]).reshape(-1, 512).numpy()
    q = torch.randn((1, H, 576), generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    qb = q.view(torch.int16).numpy().astype(np.uint16)
    # a single valid row: output equals that row's V
    locs = np.array([[-1, 9, -1]], np.int32)
    got = oracle_sparse_mla_decode(qb, locs, pool.numpy(), scale)
    assert np.allclose(got[0], np.broadcast_to(deq[9], (H, 512)), rtol=0, atol=1e-15)
    # q = 0: uniform weights, output is the mean of V
    zq = np.zeros((1, H, 576), np.uint16)
    locs = np.array([[1, 2, 3, 40, -1, 63]], np.int32)
    got = oracle_sparse_mla_decode(zq, locs, pool.numpy(), scale)
    assert np.allclose(got[0], np.broadcast_to(deq[[1, 2, 3, 40, 63]].mean(0), (H, 512)),
                       rtol=1e-13, atol=1e-13)
    # no valid row: zero output
    got = oracle_sparse_mla_decode(qb, np.full((1, 5), -1, np.int32), pool.numpy(), scale)
    assert (got == 0).all()


def test_fast_path_boundary():
    """seq_len <= device buffer size takes the fast path (slot == position,
    no copy), as stated in the per-step flow of the gogongxt.com HiSparse
    page; seq_len = S + 1 takes the LRU path (cold: j-th miss -> slot j)."""
    S, k = 16, 6
    for n, fast in [(S, True), (S + 1, False)]:
        st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
        locs = np.arange(n, dtype=np.int64)[None, :]
        host = _host_pool(n)
        row = np.array([[n - 1, 3, 0, 9, -1, 5]], np.int32)
        out = oracle_resolve(st, page_size=0, max_seq_len=n, resident_pages=0, req_idx=[0],
                             top_k_tokens=row, seq_lens=[n], host_cache_locs=locs,
                             block_table=None, host_pools=host, host_pool_rows=[n])
        if fast:
            assert out[0].tolist() == [n - 1, 3, 0, 9, -1, 5]
            assert st.stats.tolist() == [0, 0, 0, 5, 0]
            assert (st.dev_pools[0] == 0).all()          # nothing copied
        else:
            assert out[0].tolist() == [0, 1, 2, 3, -1, 4]
            assert st.stats.tolist() == [0, 5, 0, 0, 0]
