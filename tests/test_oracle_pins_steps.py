"""Pins of the multi-step (speculative decoding) reading on the oracle.

The verification steps of one decode step are consecutive resolver calls
sharing the hot state ("vLLM Hybrid HiSparse 源码实现分析" section 7.4).  With
S >= steps * k every victim of a later step is older than the whole call,
so no step evicts a row an earlier step returned; with a smaller S that can
fail, which the counterexample shows.
"""
import numpy as np

from oracle import OracleState, oracle_resolve

RB = 16


def _run(S, k, Q, decode_steps, seed):
    rng = np.random.default_rng(seed)
    n = 5000
    st = OracleState(R=1, S=S, L=1, row_bytes=RB, dev_pool_rows=S)
    locs = np.arange(n, dtype=np.int64)[None, :]
    host = [np.zeros((n, RB), np.uint8)]
    evicted = 0
    for _ in range(decode_steps):
        outs = []
        for q in range(Q):
            top = rng.choice(n, size=k, replace=False).astype(np.int32)[None]
            out = oracle_resolve(st, page_size=0, max_seq_len=n, resident_pages=0, req_idx=[0],
                                 top_k_tokens=top, seq_lens=[n], host_cache_locs=locs,
                                 block_table=None, host_pools=host, host_pool_rows=[n])
            outs.append((top[0], out[0]))
        for top, out in outs:      # after all steps: every returned row still holds its token
            evicted += int((st.slot_tokens[0, out] != top).sum())
    return evicted


def test_steps_never_evict_rows_of_earlier_steps():
    for seed in range(4):
        assert _run(S=4 * 24, k=24, Q=4, decode_steps=6, seed=seed) == 0        # S = Q k
        assert _run(S=5 * 24, k=24, Q=4, decode_steps=6, seed=seed) == 0        # (Q+1) k


def test_steps_can_evict_when_the_buffer_is_too_small():
    assert _run(S=3 * 24, k=24, Q=4, decode_steps=6, seed=0) > 0
