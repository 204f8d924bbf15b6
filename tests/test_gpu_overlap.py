"""The overlapped per-layer copy + decode gives bit-identical results to the
sequential order (plan, copy of every layer, decode of every layer), and
matches the oracle's attention within tolerance."""
import math

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from oracle import oracle_sparse_mla_decode
from tests.harness import Pair, make_host_pools
from workloads import make_queries, synth

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(192.0)


# Layer counts 1 (no copy or combine beside any decode), 2, 3 and 5 (the
# split partials alternate between two workspace halves, so odd and even
# counts end on different halves); 260 batch rows of one key split each make
# the decode alone fill the CUs, so the copy and combine workgroups of each
# launch run after it.  The last two: padding batch rows among the requests,
# and 144 heads (a full and a partial head group of 128).
@pytest.mark.parametrize("B,L,corrupt,pad,H", [(4, 3, False, 0, 32), (9, 3, False, 0, 32),
                                               (9, 3, True, 0, 32), (5, 1, False, 0, 32),
                                               (6, 2, True, 0, 32), (7, 5, False, 0, 32),
                                               (260, 2, False, 0, 32), (8, 3, False, 3, 144),
                                               (3, 2, True, 2, 144)])
def test_overlapped_layers_match_sequential(B, L, corrupt, pad, H):
    """With `corrupt`, some host rows are out of range (negative or past the
    pool), so the layer copy's zero fill and tripwire count are compared
    too."""
    print("[overlap] B=%d L=%d corrupt=%s pad=%d H=%d" % (B, L, corrupt, pad, H), flush=True)
    n0 = [3000 + 700 * b for b in range(B)] if B <= 64 else [600 + 7 * b for b in range(B)]
    w = synth("ovl", 70 + B, R=B, S=256, k=128, steps=3, n0=n0, L=L, grow=1, keep=80, recent=16,
              recent_window=64, padding_rows=pad)
    if corrupt:   # every request is past S, so admission copies no host rows
        rng = np.random.default_rng(12)
        locs = w.host_cache_locs
        locs[rng.random(locs.shape) < 0.04] = -3
        locs[rng.random(locs.shape) < 0.04] = w.host_pool_rows + 7
    bufs = make_host_pools(w, kind="mla")
    seq = Pair(w, bufs, with_oracle=False, max_heads=H)
    ovl = Pair(w, bufs, max_heads=H)
    try:
        qs = [make_queries(w.B, H, seed=10 + l, device="cuda") for l in range(L)]
        for step in range(w.steps):
            outs_s = [torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
            outs_o = [torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
            for p in (seq, ovl):
                p.pre_step_writes(step)
                hs.hisparse_resolve_plan(p.pool, None, w.B, w.k, p.req_idx, p.topk[step],
                                         p.seq[step], p.locs, p.bt, p.st, p.lru, p.clk, p.out,
                                         p.stats)
            hs.hisparse_gather_copy(seq.pool, None, w.B, 0, L, seq.stats)
            for l in range(L):
                hs.hisparse_sparse_mla_decode(seq.pool, None, w.B, H, w.k, l, qs[l], seq.out, SCALE,
                                              outs_s[l])
            hs.hisparse_decode_layers_overlapped(ovl.pool, None, w.B, H, w.k, qs, ovl.out, SCALE,
                                                 outs_o, ovl.stats)
            torch.cuda.synchronize()
            assert torch.equal(seq.out, ovl.out)
            for l in range(L):
                assert torch.equal(outs_s[l], outs_o[l]), "step %d layer %d" % (step, l)
                assert torch.equal(seq.dev_pools[l], ovl.dev_pools[l])
            assert torch.equal(seq.stats, ovl.stats)
            # the overlapped outputs are the attention of the resolved rows
            o_out = ovl.oracle_step(step, *ovl.writes_of(step))
            assert np.array_equal(ovl.out.cpu().numpy(), o_out)
            l = step % L
            ref = oracle_sparse_mla_decode(qs[l].cpu().view(torch.int16).numpy().astype(np.uint16),
                                           o_out, ovl.ost.dev_pools[l], float(np.float32(SCALE)))
            got = outs_o[l].float().cpu().numpy().astype(np.float64)
            err = np.abs(got - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)
            print("[overlap] step %d layer %d max normwise error %.3g" % (step, l, err.max()),
                  flush=True)
            assert err.max() <= 2e-2
        if corrupt:
            assert int(ovl.stats[4].item()) > 0
    finally:
        seq.close()
        ovl.close()


def test_overlapped_rejects_bad_layer_before_enqueueing():
    """Every layer's arguments are checked before anything is enqueued: a
    misaligned query of the last layer is refused (EINVAL) and no layer's
    device pool or the stats have changed (layer 0's copy never ran)."""
    import ctypes
    print("[overlap] bad last layer", flush=True)
    L, H, B = 3, 32, 4
    w = synth("ovl_bad", 91, R=B, S=256, k=128, steps=1, n0=[3000, 3500, 4000, 4500], L=L)
    pair = Pair(w, make_host_pools(w, kind="mla"), with_oracle=False, max_heads=H)
    try:
        pair.pre_step_writes(0)
        hs.hisparse_resolve_plan(pair.pool, None, w.B, w.k, pair.req_idx, pair.topk[0], pair.seq[0],
                                 pair.locs, pair.bt, pair.st, pair.lru, pair.clk, pair.out, pair.stats)
        torch.cuda.synchronize()
        before = [d.clone() for d in pair.dev_pools]
        stats_before = pair.stats.clone()
        qs = [make_queries(w.B, H, seed=l, device="cuda") for l in range(L)]
        outs = [torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
        qp = (ctypes.c_void_p * L)(*[q.data_ptr() for q in qs])
        qp[L - 1] = qs[L - 1].data_ptr() + 2          # not 16-byte aligned
        op = (ctypes.c_void_p * L)(*[o.data_ptr() for o in outs])
        lib = hs.load_library()
        rc = lib.hisparse_decode_layers_overlapped(
            ctypes.c_void_p(pair.pool.handle), None, w.B, H, w.k, ctypes.cast(qp, ctypes.c_void_p),
            ctypes.c_void_p(pair.out.data_ptr()), ctypes.c_float(SCALE),
            ctypes.cast(op, ctypes.c_void_p), ctypes.c_void_p(pair.stats.data_ptr()))
        torch.cuda.synchronize()
        assert rc == -1 and "aligned" in hs.hisparse_last_error()
        for l in range(L):
            assert torch.equal(before[l], pair.dev_pools[l]), "layer %d changed" % l
        assert torch.equal(stats_before, pair.stats)
    finally:
        pair.close()
