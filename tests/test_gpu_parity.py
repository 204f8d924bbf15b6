"""GPU parity of the HIP resolver against the CPU oracle (bit-exact).

Every step compares device_buffer_locs, slot_tokens, lru_slots, lru_clock,
the five counters and the device rows named by that step's output; the
whole device pools are compared at the end.  Calls go through the C ABI
(ctypes binding of libhisparse.so).
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from tests.harness import Pair, make_host_pools, run_parity
from workloads import synth, config1_tiny

pytestmark = pytest.mark.gpu


def _log(name):
    def f(step):
        if step % 8 == 0:
            print("[%s] step %d ok" % (name, step), flush=True)
    return f


def test_config1_tiny_all_steps():
    print("[config1] 4 req, n=8192, k=256, S=512, 32 steps", flush=True)
    w = config1_tiny()
    stats = run_parity(w, log=_log("config1"))
    assert stats[1] > 0 and stats[0] > 0


# Batches of 8 or more take the copy inside the plan kernel through
# hisparse_resolve; "split" runs the same steps through the plan and copy
# entry points.
MODES = ["resolve", "split"]


@pytest.mark.parametrize("mode", MODES)
def test_ragged_shapes_fast_path_transition_and_padding(mode):
    """S and k not multiples of the wavefront or block size, padding rows,
    fast-path rows that cross seq_len == S during the run, rows with
    seq_len <= k (padded top-k)."""
    print("[ragged %s] S=200 k=77 steps=8" % mode, flush=True)
    w = synth("ragged", 21, R=7, S=200, k=77, steps=8,
              n0=[1000, 300, 198, 200, 5000, 60], grow=1, keep=50, recent=10,
              recent_window=100, padding_rows=2)
    run_parity(w, log=_log("ragged"), mode=mode)


@pytest.mark.parametrize("mode", MODES)
def test_multi_layer_shared_plan(mode):
    print("[layers %s] L=3" % mode, flush=True)
    w = synth("layers", 22, R=10, S=256, k=128, steps=6,
              n0=[4000, 3000, 2500, 9000, 700, 1200, 5000, 3300, 260], L=3,
              keep=100, recent=8, recent_window=64)
    run_parity(w, log=_log("layers"), mode=mode)


def test_more_layers_than_the_fused_copy_takes():
    """Nine layers: hisparse_resolve falls back to the separate copy kernel."""
    print("[layers] L=9", flush=True)
    w = synth("layers9", 28, R=8, S=128, k=64, steps=3, n0=[900, 700, 500, 2000, 300, 150, 1000, 640],
              L=9, keep=40)
    run_parity(w, log=_log("layers9"))


@pytest.mark.parametrize("mode", MODES)
def test_resident_pages_small(mode):
    print("[resident %s] P=16 tail=256" % mode, flush=True)
    w = synth("resident", 23, R=8, S=256, k=128, steps=6, n0=[2048] * 8, keep=90,
              P=16, resident_tail=256)
    stats = run_parity(w, log=_log("resident"), mode=mode)
    assert stats[2] > 0


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("P,tail", [(1, 256), (24, 240), (100, 300)])
def test_resident_page_sizes(mode, P, tail):
    """Single-token pages and page sizes that are not powers of two (the
    block-table lookup then divides instead of shifting), on rows that grow
    every step, with a padding row."""
    print("[resident %s] P=%d tail=%d" % (mode, P, tail), flush=True)
    w = synth("pages%d" % P, 31 + P, R=8, S=256, k=128, steps=5,
              n0=[2048, 3000, 1000, 5000, 700, 4096, 2500, 6000], grow=7, keep=90,
              P=P, resident_tail=tail, padding_rows=1)
    stats = run_parity(w, mode=mode)
    assert stats[2] > 0


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("S", [1, 2])
def test_smallest_hot_buffers(mode, S):
    """One or two hot slots with top-k = S: rows of 1 token (fast path), rows
    that leave it, long rows where every step's miss evicts the previous
    token, a padding row; nine rows, so the single-call entry point fuses."""
    print("[smallest %s] S=k=%d" % (mode, S), flush=True)
    w = synth("tiny%d" % S, 61 + S, R=9, S=S, k=S, steps=6,
              n0=[1, S, S + 1, 40, 900, 2, 7, 3000, 1], grow=1, keep=S // 2, padding_rows=1)
    stats = run_parity(w, mode=mode)
    assert stats[1] > 0 and stats[3] > 0  # misses, and fast-path entries


@pytest.mark.parametrize("mode", MODES)
def test_top_k_equals_slots(mode):
    print("[k=S %s] S=k=2048" % mode, flush=True)
    w = synth("kS", 24, R=8, S=2048, k=2048, steps=4,
              n0=[50000, 40000, 30000, 9000, 2100, 2048, 70000, 12345], keep=1800)
    run_parity(w, log=_log("k=S"), mode=mode)


def _table_bucket(t, nbk):
    """The bucket a position hashes to in the resolver's table of nbk buckets
    (Knuth's multiplicative hash, top log2(nbk) bits of the 32-bit product)."""
    t = np.asarray(t, dtype=np.uint64)
    return ((t * np.uint64(2654435761)) & np.uint64(0xFFFFFFFF)) >> np.uint64(32 - int(np.log2(nbk)))


@pytest.mark.parametrize("mode", MODES)
def test_table_bucket_overflow_and_wraparound(mode):
    """Every step each row's top-k starts with 60 positions drawn from the
    ones that hash into the table's last two buckets, so inserts overflow
    across a chain of buckets that wraps past the table's end, and probes
    walk it.  The draws overlap from step to step, so slots hold some of
    those positions as hits and others that are not pending (probes that
    must end absent).  The table shape assumed is the kernel's at S=512,
    k=256: 8 cells per entry in buckets of 4, 512 buckets.  Were it another,
    the comparison would still be bit-exact, only the stress weaker."""
    print("[collide %s] S=512 k=256" % mode, flush=True)
    S, k, n = 512, 256, 60000
    w = synth("collide", 71, R=8, S=S, k=k, steps=5, n0=[n] * 8, keep=128)
    nbk = 8 * k // 4
    pos = np.arange(n, dtype=np.int64)
    bk = _table_bucket(pos, nbk)
    pool = np.concatenate([pos[bk == nbk - 1], pos[bk == nbk - 2]])
    assert len(pool) >= 200
    rng = np.random.default_rng(17)
    for step in range(w.steps):
        for b in range(w.B):
            hot = rng.choice(pool, size=60, replace=False).tolist()
            taken = set(hot)
            rest = [int(x) for x in w.top_k[step, b] if x >= 0 and int(x) not in taken]
            w.top_k[step, b] = np.array(hot + rest[:k - 60], dtype=np.int32)
    stats = run_parity(w, log=_log("collide"), mode=mode)
    assert stats[0] > 0 and stats[1] > 0


def test_zero_top_k_and_empty_batch():
    w = synth("k0", 25, R=2, S=64, k=8, steps=1, n0=[500, 100])
    bufs = make_host_pools(w)
    pair = Pair(w, bufs)
    try:
        empty = torch.empty((w.B, 0), dtype=torch.int32, device="cuda")
        hs.hisparse_resolve(pair.pool, None, w.B, 0, pair.req_idx, empty, pair.seq[0], pair.locs,
                            None, pair.st, pair.lru, pair.clk, empty, pair.stats)
        e1 = torch.empty((0,), dtype=torch.int32, device="cuda")
        hs.hisparse_resolve(pair.pool, None, 0, w.k, e1, torch.empty((0, w.k), dtype=torch.int32,
                            device="cuda"), e1, pair.locs, None, pair.st, pair.lru, pair.clk,
                            torch.empty((0, w.k), dtype=torch.int32, device="cuda"), pair.stats)
        torch.cuda.synchronize()
        assert pair.clk.cpu().tolist() == [1, 1]          # one active call each
        assert pair.stats.cpu().tolist() == [0, 0, 0, 0, 0]
    finally:
        pair.close()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("layers", [1, 2])
def test_corrupt_state_and_tripwires(mode, layers):
    """Corrupt slot map (markers below -1, one position in two slots, tokens
    past seq_len), scrambled stamps (forces the full-sort victim path),
    out-of-range host rows and block-table ids, a request index past R."""
    print("[corrupt %s L=%d]" % (mode, layers), flush=True)
    w = synth("corrupt", 26, R=9, S=96, k=40, steps=5,
              n0=[3000, 2000, 1500, 800, 4000, 90, 2500, 1200], L=layers,
              keep=30, P=8, resident_tail=64, padding_rows=1)
    rng = np.random.default_rng(5)
    w.req_idx[w.req_idx < 0] = w.R + 2
    bufs = make_host_pools(w)
    pair = Pair(w, bufs, mode=mode)      # admission uses the clean tables
    try:
        locs = w.host_cache_locs
        locs[rng.random(locs.shape) < 0.05] = -7
        locs[rng.random(locs.shape) < 0.05] = w.host_pool_rows + 3
        bt = w.block_table
        bt[(bt >= 0) & (rng.random(bt.shape) < 0.2)] = w.resident_pages + 1
        pair.locs.copy_(torch.from_numpy(locs))
        pair.bt.copy_(torch.from_numpy(bt))
        st = rng.integers(-4, 3500, size=(w.R, w.S)).astype(np.int32)
        st[0, 3] = st[0, 70] = 1234
        lru = rng.permutation(w.R * w.S).reshape(w.R, w.S).astype(np.int32) - 200
        pair.st.copy_(torch.from_numpy(st))
        pair.lru.copy_(torch.from_numpy(lru))
        pair.ost.slot_tokens[:] = st
        pair.ost.lru_slots[:] = lru
        for step in range(w.steps):
            dst, src = pair.gpu_step(step)
            o = pair.oracle_step(step, dst, src)
            torch.cuda.synchronize()
            pair.compare_step(step, o)
        pair.compare_pools()
        assert pair.ost.stats[4] > 0
    finally:
        pair.close()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("spread", [1, 20, 80, 130, 200, 400])
def test_victim_keys_spread_over_windows(mode, spread):
    """Victims are ranked by windows of up to 32 consecutive keys above the
    smallest remaining one.  Here every request starts with about 3% empty
    slots whose stamps are 0, 1 or 2 (their own window, first) and occupied
    slots whose stamps take `spread` consecutive values, so the first step's
    ~235 victims per request need two windows (spread 1, 20), three (80),
    three or four (130), four or five (200) or seven or eight (400); beyond
    the four windows allowed the bitonic-sort fallback finishes the ranking.
    Each step must match the oracle bit for bit."""
    print("[spread %s] %d" % (mode, spread), flush=True)
    S, k = 512, 256
    n0 = [5000 + 331 * b for b in range(9)]
    w = synth("spread", 61 + spread, R=10, S=S, k=k, steps=3, n0=n0, keep=64)
    pair = Pair(w, make_host_pools(w), mode=mode)
    try:
        rng = np.random.default_rng(spread)
        st = np.empty((w.R, S), np.int32)
        lru = np.empty((w.R, S), np.int32)
        for r in range(w.R):
            st[r] = rng.choice(4000, size=S, replace=False)   # distinct valid tokens
            lru[r] = 1000 + rng.integers(0, spread, size=S)
            empty = rng.random(S) < 0.03
            st[r, empty] = -1
            lru[r, empty] = rng.integers(0, 3, size=int(empty.sum()))
        clk = np.full(w.R, 1000 + spread + 5, np.int32)
        for t, a in ((pair.st, st), (pair.lru, lru), (pair.clk, clk)):
            t.copy_(torch.from_numpy(a))
        pair.ost.slot_tokens[:], pair.ost.lru_slots[:], pair.ost.lru_clock[:] = st, lru, clk
        for step in range(w.steps):
            dst, src = pair.gpu_step(step)
            o = pair.oracle_step(step, dst, src)
            torch.cuda.synchronize()
            pair.compare_step(step, o)
        pair.compare_pools()
        assert pair.ost.stats[1] > 0
    finally:
        pair.close()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("S,k", [(4096, 4096), (8192, 4096), (16384, 2004)])
def test_lds_budget_corners(mode, S, k):
    """The largest slot / top-k pairs the LDS budget allows: the table with
    two cells per entry, 4 and 8 top-k entries and 4, 8 and 16 slots per
    thread.  After the cold step the stamps are scrambled, so step 1 ranks
    its victims through the full sort over every slot."""
    print("[corner %s] S=%d k=%d" % (mode, S, k), flush=True)
    n0 = [2 * S + 7, 3 * S, 2 * S + 100, 4 * S, 2 * S + 33, 3 * S - 1, 5 * S, 2 * S + 1]
    w = synth("corner", 29, R=8, S=S, k=k, steps=3, n0=n0, keep=(3 * k) // 4)
    bufs = make_host_pools(w)
    pair = Pair(w, bufs, mode=mode)
    try:
        rng = np.random.default_rng(9)
        for step in range(w.steps):
            if step == 1:
                lru = (rng.permutation(w.R * w.S).reshape(w.R, w.S) - 1000).astype(np.int32)
                pair.lru.copy_(torch.from_numpy(lru))
                pair.ost.lru_slots[:] = lru
            dst, src = pair.gpu_step(step)
            o = pair.oracle_step(step, dst, src)
            torch.cuda.synchronize()
            pair.compare_step(step, o)
            print("[corner %s] S=%d k=%d step %d ok" % (mode, S, k, step), flush=True)
        pair.compare_pools()
        assert pair.ost.stats[1] > 0
    finally:
        pair.close()


def test_host_side_errors():
    w = synth("err", 27, R=2, S=64, k=8, steps=1, n0=[500, 100])
    bufs = make_host_pools(w)
    pair = Pair(w, bufs, with_oracle=False)
    try:
        big = torch.zeros((w.B + 5, w.k), dtype=torch.int32, device="cuda")
        with pytest.raises(ValueError):     # shape check in the binding
            hs.hisparse_resolve(pair.pool, None, w.B, w.k, pair.req_idx, big, pair.seq[0],
                                pair.locs, None, pair.st, pair.lru, pair.clk, pair.out, None)
        lib = hs.load_library()
        import ctypes
        rc = lib.hisparse_resolve(ctypes.c_void_p(pair.pool.handle), None, w.B + 100, w.k,
                                  *([None] * 10))
        assert rc == -1 and "max_batch" in hs.hisparse_last_error()
        rc = lib.hisparse_gather_copy(ctypes.c_void_p(pair.pool.handle), None, w.B, 0, 5, None)
        assert rc == -1
        # a host pool that is not pinned memory is refused at init
        plain = np.zeros((w.host_pool_rows, 656), np.uint8)
        cfg = hs.PoolConfig(max_requests=w.R, slots=w.S, max_top_k=w.k, max_batch=w.B,
                            max_seq_len=w.max_seq_len)
        with pytest.raises(hs.HisparseError):
            hs.hisparse_init_pool(cfg, [plain.ctypes.data], [w.host_pool_rows],
                                  pair.dev_pools, w.dev_pool_rows)
        bad = hs.PoolConfig(max_requests=w.R, slots=w.S, max_top_k=w.S + 1, max_batch=w.B,
                            max_seq_len=w.max_seq_len)
        with pytest.raises(hs.HisparseError):
            hs.hisparse_init_pool(bad, bufs, [w.host_pool_rows], pair.dev_pools, w.dev_pool_rows)
        # the pool still works after the refused calls
        pair.gpu_step(0)
        torch.cuda.synchronize()
    finally:
        pair.close()


def test_copy_batch_must_match_the_plan():
    """A copy replays the compact plan of the last plan call: before any plan,
    or with a batch other than the plan's, the copy entry points refuse
    (EINVAL) instead of replaying rows of an older plan; so does a decode of
    more heads than the pool's max_heads or more rows than its max_batch.
    The pool then runs a normal step, checked against the oracle."""
    import ctypes
    print("[copy batch check]", flush=True)
    w = synth("cbatch", 29, R=4, S=64, k=8, steps=2, n0=[500, 700, 900, 300])
    pair = Pair(w, make_host_pools(w), mode="split", max_heads=16)
    lib = hs.load_library()
    h = ctypes.c_void_p(pair.pool.handle)
    try:
        rc = lib.hisparse_gather_copy(h, None, w.B, 0, 1, None)
        assert rc == -1 and "no plan" in hs.hisparse_last_error()
        dst, src = pair.gpu_step(0)          # plan of batch w.B, then its copy
        o = pair.oracle_step(0, dst, src)
        rc = lib.hisparse_gather_copy(h, None, w.B - 1, 0, 1, None)
        assert rc == -1 and "differs" in hs.hisparse_last_error()
        rc = lib.hisparse_gather_copy_step(h, None, 0, w.B + 0, 0, 1, None)
        assert rc == 0, hs.hisparse_last_error()   # same batch: a valid replay
        rc = lib.hisparse_gather_copy_step(h, None, 0, 2, 0, 1, None)
        assert rc == -1 and "differs" in hs.hisparse_last_error()
        q = torch.zeros((w.B, 32, 576), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((w.B, 32, 512), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(hs.HisparseError, match="max_heads"):
            hs.hisparse_sparse_mla_decode(pair.pool, None, w.B, 32, w.k, 0, q, pair.out, 1.0, out)
        rc = lib.hisparse_sparse_mla_decode(h, None, w.B + 1, 16, w.k, 0,
                                            ctypes.c_void_p(q.data_ptr()),
                                            ctypes.c_void_p(pair.out.data_ptr()), ctypes.c_float(1.0),
                                            ctypes.c_void_p(out.data_ptr()))
        assert rc == -1 and "max_batch" in hs.hisparse_last_error()
        torch.cuda.synchronize()
        pair.compare_step(0, o)
        dst, src = pair.gpu_step(1)
        o = pair.oracle_step(1, dst, src)
        torch.cuda.synchronize()
        pair.compare_step(1, o)
    finally:
        pair.close()


def test_pool_holds_its_buffers():
    """The library keeps raw pointers to the device pools and host buffers,
    so the binding's pool object keeps them alive until it is destroyed: a
    caller that drops its own references must not leave the kernels writing
    into memory handed out again."""
    import gc
    import weakref
    hb = hs.HostBuffer(656 * 64)
    dev = torch.zeros((64, 656), dtype=torch.uint8, device="cuda")
    refs = (weakref.ref(hb), weakref.ref(dev))
    cfg = hs.PoolConfig(max_requests=1, slots=64, max_top_k=16, max_batch=1, max_seq_len=64)
    pool = hs.hisparse_init_pool(cfg, [hb], [64], [dev], 64)
    del hb, dev
    gc.collect()
    assert all(r() is not None for r in refs)
    hs.hisparse_destroy_pool(pool)
    gc.collect()
    assert all(r() is None for r in refs)


@pytest.mark.parametrize("mode", MODES)
def test_duplicate_positions_are_safe(mode):
    """Distinct positions per row are a caller precondition; with repeats the
    results are unspecified (the oracle and the kernel may place a repeat
    differently), but the kernel must finish, emit only row IDs inside the
    device pool (or -1), copy only into hot rows, and keep working on the
    in-contract steps that follow."""
    print("[duplicates %s]" % mode, flush=True)
    w = synth("dups", 27, R=10, S=128, k=48, steps=6, n0=[3000, 2500, 900, 4000, 5000, 1200, 3500,
                                                          2800, 700, 6000], keep=30)
    pair = Pair(w, make_host_pools(w), with_oracle=False, mode=mode)
    try:
        rng = np.random.default_rng(27)
        for step in range(w.steps):
            if step in (1, 3):   # repeat some valid positions inside their rows
                tk = w.top_k[step].copy()
                for b in range(w.B):
                    src = rng.choice(w.k, size=6, replace=False)
                    dst = rng.choice(w.k, size=6, replace=False)
                    tk[b, dst] = tk[b, src]
                pair.topk[step].copy_(torch.from_numpy(tk))
            pair.gpu_step(step)
            torch.cuda.synchronize()
            out = pair.out.cpu().numpy()
            assert ((out == -1) | ((out >= 0) & (out < w.dev_pool_rows))).all(), "step %d" % step
            st = pair.st.cpu().numpy()
            assert ((st >= -1) & (st < w.max_seq_len)).all()
        stats = pair.stats.cpu().numpy()
        assert stats[0] > 0 and stats[1] > 0 and stats[4] == 0
    finally:
        pair.close()


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("row_bytes", [16, 1040, 2064])
def test_row_widths(mode, row_bytes):
    """Rows of any multiple of 16 bytes: one 16-byte unit, and rows of 65
    and 129 units, more than one unit per lane (the fused instance then
    skips its early loads of the first layer's rows and every lane copies
    several units).  Two layers, fast-path and LRU rows and a padding row;
    every step's named rows and the whole pools are compared."""
    print("[row widths %s %d]" % (mode, row_bytes), flush=True)
    w = synth("rows%d" % row_bytes, 77 + row_bytes, R=12, S=256, k=96, steps=4,
              n0=[300, 700, 1500, 90, 2000, 256, 1200, 5000, 640, 3000], L=2, grow=3,
              keep=60, recent=16, recent_window=90, padding_rows=1)
    w.row_bytes = row_bytes
    stats = run_parity(w, mode=mode)
    assert stats[1] > 0  # misses were copied


def test_largest_batch():
    """The largest batch a pool admits (65,535 rows, one workgroup each),
    with 5 padding rows among them and one-unit rows to keep the pools small:
    two steps through the single-call entry point, bit-exact."""
    B, pad = 65535, 5
    rng = np.random.default_rng(5)
    n0 = [int(v) for v in rng.integers(1, 64, size=B - pad)]
    print("[largest batch %d]" % B, flush=True)
    w = synth("maxbatch", 90, R=B - pad, S=16, k=8, steps=2, n0=n0, grow=1, keep=5,
              recent=1, recent_window=1, padding_rows=pad)
    w.row_bytes = 16
    assert w.B == 65535
    stats = run_parity(w)
    assert stats[1] > 0
