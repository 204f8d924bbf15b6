"""Pins of the oracle's row mirror and hot-entry invalidation (CPU only).

The mirror is pinned by a hand-worked example and by a round trip through
the resolver back to the bytes that were written; the invalidations by an
independent numpy formulation (set membership over the whole state) and by
their effect on the next resolver call (exactly the cleared tokens miss).
"""
import numpy as np
import pytest

from oracle import (OracleState, oracle_invalidate_host_rows, oracle_invalidate_tokens,
                    oracle_mirror_rows, oracle_resolve)

RB = 16


def test_mirror_worked_example():
    """Two layers, device rows filled with their own index; entries: device
    row 2 -> host row 5, a padding entry, device row 9 (past the 8-row pool)
    -> host row 3, device row 4 -> host row 10 (one past the 10-row host pool;
    the arrays hold 12 rows so that a copy there would be seen)."""
    st = OracleState(R=1, S=8, L=2, row_bytes=RB, dev_pool_rows=8)
    for l in range(2):
        st.dev_pools[l][:] = (np.arange(8, dtype=np.uint8)[:, None] + 16 * l)
    host = [np.full((12, RB), 0xEE, np.uint8) for _ in range(2)]
    oracle_mirror_rows(st, dev_rows=[2, -1, 9, 4], host_rows=[5, 7, 3, 10], host_pools=host,
                       host_pool_rows=[10, 10])
    for l in range(2):
        assert (host[l][5] == 2 + 16 * l).all()
        untouched = [r for r in range(12) if r != 5]
        assert (host[l][untouched] == 0xEE).all()
    assert st.stats[4] == 4           # two bad entries x two layers
    # a layer range copies only those layers
    host2 = [np.zeros((10, RB), np.uint8) for _ in range(2)]
    oracle_mirror_rows(st, dev_rows=[3], host_rows=[1], host_pools=host2, host_pool_rows=[10, 10],
                       layer_begin=1, layer_end=2)
    assert (host2[0] == 0).all() and (host2[1][1] == 3 + 16).all()


def test_mirror_rejects_duplicate_destinations_when_validating():
    st = OracleState(R=1, S=4, L=1, row_bytes=RB, dev_pool_rows=4)
    host = [np.zeros((8, RB), np.uint8)]
    with pytest.raises(ValueError):
        oracle_mirror_rows(st, dev_rows=[0, 1], host_rows=[3, 3], host_pools=host,
                           host_pool_rows=[8], validate=True)
    # a padding entry does not count as a destination
    oracle_mirror_rows(st, dev_rows=[0, -1], host_rows=[3, 3], host_pools=host,
                       host_pool_rows=[8], validate=True)


def test_mirror_then_resolve_round_trip():
    """Rows written on the device by the forward pass of a fast-path request,
    mirrored to the host, come back byte for byte when a fresh buffer
    resolves them on the LRU path."""
    rng = np.random.default_rng(3)
    S, n = 16, 12
    locs = rng.permutation(40)[:n].astype(np.int64)[None, :]   # host row of each token
    written = rng.integers(0, 256, size=(n, RB), dtype=np.uint8)
    st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
    st.dev_pools[0][:n] = written                                # fast path: slot == token
    host = [np.zeros((40, RB), np.uint8)]
    oracle_mirror_rows(st, dev_rows=np.arange(n), host_rows=locs[0], host_pools=host,
                       host_pool_rows=[40], validate=True)
    fresh = OracleState(R=1, S=4, L=1, row_bytes=RB, dev_pool_rows=4)
    top = np.array([[7, 2, 11, 0]], np.int32)
    out = oracle_resolve(fresh, page_size=0, max_seq_len=n, resident_pages=0, req_idx=[0],
                         top_k_tokens=top, seq_lens=[n], host_cache_locs=locs, block_table=None,
                         host_pools=host, host_pool_rows=[40])
    for i, t in enumerate(top[0]):
        assert (fresh.dev_pools[0][out[0, i]] == written[t]).all()


def _random_state(rng, R, S, n):
    st = OracleState(R=R, S=S, L=1, row_bytes=RB, dev_pool_rows=R * S)
    for r in range(R):
        occ = rng.random(S) < 0.8
        st.slot_tokens[r] = np.where(occ, rng.permutation(n)[:S], -1)
        st.lru_slots[r] = np.where(occ, rng.integers(1, 50, S), 0)
    st.slot_tokens[0, 0] = -3                                    # a corrupted empty marker
    return st


@pytest.mark.parametrize("seed", range(6))
def test_invalidate_tokens_vs_numpy(seed):
    rng = np.random.default_rng(seed)
    R, S, n = 5, 24, 100
    st = _random_state(rng, R, S, n)
    st0, lru0 = st.slot_tokens.copy(), st.lru_slots.copy()
    req = np.array([3, -1, 0, 7, 3], np.int32)                   # padding, out of range, repeat
    b = rng.integers(0, n, 5).astype(np.int32)
    e = (b + rng.integers(0, 30, 5)).astype(np.int32)
    oracle_invalidate_tokens(st, req_rows=req, tok_begin=b, tok_end=e)
    exp_t, exp_l = st0.copy(), lru0.copy()
    for r, lo, hi in zip(req, b, e):
        if 0 <= r < R:
            hit = (exp_t[r] >= lo) & (exp_t[r] < hi)
            exp_t[r][hit] = -1
            exp_l[r][hit] = 0
    assert np.array_equal(st.slot_tokens, exp_t) and np.array_equal(st.lru_slots, exp_l)
    assert st.stats[4] == 1


@pytest.mark.parametrize("seed", range(6))
def test_invalidate_host_rows_vs_numpy(seed):
    rng = np.random.default_rng(10 + seed)
    R, S, n = 4, 20, 60
    st = _random_state(rng, R, S, n)
    st0, lru0 = st.slot_tokens.copy(), st.lru_slots.copy()
    locs = rng.permutation(R * n).reshape(R, n).astype(np.int64)
    rows = np.sort(rng.choice(R * n, size=25, replace=False)).astype(np.int64)
    oracle_invalidate_host_rows(st, rows=rows, host_cache_locs=locs, max_seq_len=n, validate=True)
    tok = st0
    valid = (tok >= 0) & (tok < n)
    h = np.where(valid, np.take_along_axis(locs, np.clip(tok, 0, n - 1), axis=1), -1)
    hit = valid & np.isin(h, rows)
    assert np.array_equal(st.slot_tokens, np.where(hit, -1, st0))
    assert np.array_equal(st.lru_slots, np.where(hit, 0, lru0))


def test_invalidate_host_rows_rejects_unsorted_when_validating():
    st = OracleState(R=1, S=4, L=1, row_bytes=RB, dev_pool_rows=4)
    with pytest.raises(ValueError):
        oracle_invalidate_host_rows(st, rows=[5, 2], host_cache_locs=np.zeros((1, 8), np.int64),
                                    max_seq_len=8, validate=True)


def test_invalidated_tokens_miss_and_refetch_new_content():
    """After some host rows are rewritten and invalidated, the next call
    misses on exactly those tokens and copies the new bytes; the rest hit."""
    rng = np.random.default_rng(21)
    S, k, n = 32, 16, 200
    locs = np.arange(n, dtype=np.int64)[None, :]
    host = [rng.integers(0, 256, size=(n, RB), dtype=np.uint8)]
    st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
    top = rng.choice(n, size=k, replace=False).astype(np.int32)[None]
    kw = dict(page_size=0, max_seq_len=n, resident_pages=0, req_idx=[0], seq_lens=[n],
              host_cache_locs=locs, block_table=None, host_pools=host, host_pool_rows=[n])
    oracle_resolve(st, top_k_tokens=top, **kw)
    rewritten = np.sort(top[0, :5]).astype(np.int64)             # host rows of 5 tokens
    host[0][rewritten] = 0xAB
    oracle_invalidate_host_rows(st, rows=rewritten, host_cache_locs=locs, max_seq_len=n)
    before = st.stats.copy()
    out = oracle_resolve(st, top_k_tokens=top, **kw)
    assert st.stats[1] - before[1] == 5 and st.stats[0] - before[0] == k - 5
    for i in range(k):
        assert (st.dev_pools[0][out[0, i]] == host[0][top[0, i]]).all()
