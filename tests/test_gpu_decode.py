"""GPU parity of the sparse-MLA decode kernel against the float64 CPU oracle.

Tolerance: for every (batch row, head), max|O_gpu - O_ref| / max|O_ref| must
not exceed 2e-2 (normwise; the elementwise ratio is meaningless near zero).
"""
import math

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from oracle import oracle_sparse_mla_decode
from tests.harness import Pair, make_host_pools
from workloads import (config2_dsa_decode, fill_host_rows_mla, make_queries, synth)

pytestmark = pytest.mark.gpu
TOL = 2e-2
SCALE = 1.0 / math.sqrt(192.0)


def _normwise(got, ref):
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return np.where(den > 0, num / np.maximum(den, 1e-30), num)


def _run_decode(dev_pool, locs_np, q, heads, max_top_k, row_bytes=656):
    B, k = locs_np.shape
    hb = hs.HostBuffer(row_bytes * 16)
    cfg = hs.PoolConfig(max_requests=1, slots=max(16, max_top_k), max_top_k=max(1, max_top_k),
                        max_batch=B, max_seq_len=16, max_heads=heads, row_bytes=row_bytes)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev_pool], dev_pool.shape[0])
    try:
        locs = torch.from_numpy(locs_np).cuda()
        out = torch.empty((B, heads, 512), dtype=torch.bfloat16, device="cuda")
        hs.hisparse_sparse_mla_decode(pool, None, B, heads, k, 0, q, locs, SCALE, out)
        torch.cuda.synchronize()
        return out.float().cpu().numpy().astype(np.float64)
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


# Key splits per row at these shapes: 3, 2, 2, 10, 4, 16, 8, 16, 1 and 1, so
# the split combine runs at each of its unrolled widths (2, 4, 8, 16).  The
# last three: the largest top-k the resolver takes (4096 keys, 16 splits of 8
# blocks), one split because the batch alone fills the CUs (160 rows), and
# one split because a single ragged block holds every key.
@pytest.mark.parametrize("B,H,k", [(5, 32, 77), (3, 16, 33), (2, 48, 64), (4, 128, 300),
                                   (3, 256, 100), (1, 128, 2048), (32, 64, 256), (2, 128, 4096),
                                   (160, 128, 96), (1, 16, 20)])
def test_decode_small_vs_oracle(B, H, k):
    print("[decode] B=%d H=%d k=%d" % (B, H, k), flush=True)
    rows = max(900, k + 64)
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 31 + k, gen_device="cuda")
    rng = np.random.default_rng(k)
    locs = rng.integers(0, rows, size=(B, k)).astype(np.int32)
    locs[0, ::7] = -1                      # masked entries
    locs[-1, 3] = rows + 5                 # out of range: skipped
    if B > 2:
        locs[1, :] = -1                    # a row with nothing to attend to
        locs[1, k // 2] = 11
    q = make_queries(B, H, seed=k, device="cuda")
    got = _run_decode(dev, locs, q, H, k)
    ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                   dev.cpu().numpy(), float(np.float32(SCALE)))
    err = _normwise(got, ref)
    print("[decode] max normwise error %.3g" % err.max(), flush=True)
    assert err.max() <= TOL


@pytest.mark.parametrize("row_bytes", [672, 1024])
def test_decode_padded_rows_vs_oracle(row_bytes):
    """Rows stored at a stride above the 656-byte record (row_bytes a larger
    multiple of 16).  The bytes past the record are all 0xFF, an e4m3 NaN
    code, so reading any of them would turn outputs into NaN."""
    print("[decode padded] row_bytes=%d" % row_bytes, flush=True)
    B, H, k, rows = 3, 128, 200, 700
    rec = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(rec, 41, gen_device="cuda")
    dev = torch.full((rows, row_bytes), 0xFF, dtype=torch.uint8, device="cuda")
    dev[:, :656] = rec
    rng = np.random.default_rng(row_bytes)
    locs = rng.integers(0, rows, size=(B, k)).astype(np.int32)
    locs[0, ::5] = -1
    q = make_queries(B, H, seed=9, device="cuda")
    got = _run_decode(dev, locs, q, H, k, row_bytes=row_bytes)
    assert np.isfinite(got).all()
    ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                   dev.cpu().numpy(), float(np.float32(SCALE)), row_bytes=row_bytes)
    err = _normwise(got, ref)
    print("[decode padded] max normwise error %.3g" % err.max(), flush=True)
    assert err.max() <= TOL
    # the allocation-free entry point takes the stride from the pool tensor
    out2 = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
    hs.hisparse_sparse_mla_decode_noalloc(None, B, H, k, dev, q, torch.from_numpy(locs).cuda(),
                                          SCALE, out2)
    torch.cuda.synchronize()
    assert np.array_equal(out2.float().cpu().numpy().astype(np.float64), got)


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes_vs_oracle(seed):
    """Seeded random shapes: batch 1-4, 16-144 heads (one or two head groups,
    a partial second group), 1-300 keys, masked and out-of-range entries at a
    random rate, sometimes a row with nothing to attend to."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 5))
    H = int(rng.choice([16, 32, 48, 64, 128, 144]))
    k = int(rng.integers(1, 301))
    rows = k + int(rng.integers(16, 400))
    print("[decode random %d] B=%d H=%d k=%d rows=%d" % (seed, B, H, k, rows), flush=True)
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 600 + seed, gen_device="cuda")
    locs = rng.integers(0, rows, size=(B, k)).astype(np.int32)
    locs[rng.random((B, k)) < rng.uniform(0.0, 0.5)] = -1
    locs[rng.random((B, k)) < 0.03] = rows + 5
    if B > 1 and rng.random() < 0.5:
        locs[int(rng.integers(0, B)), :] = -1
    q = make_queries(B, H, seed=700 + seed, device="cuda")
    got = _run_decode(dev, locs, q, H, k)
    ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                   dev.cpu().numpy(), float(np.float32(SCALE)))
    err = _normwise(got, ref)
    print("[decode random %d] max normwise error %.3g" % (seed, err.max()), flush=True)
    assert err.max() <= TOL


def test_decode_score_far_above_the_first_block():
    """One key in a late block scores far above everything in the first block
    (a query aligned with that key's K vector), so the kernel's second pass
    with a higher reference runs; the result must still match."""
    print("[decode] second pass", flush=True)
    B, H, k, rows = 2, 32, 2048, 3000
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 77, gen_device="cuda")
    rng = np.random.default_rng(9)
    locs = rng.integers(0, rows, size=(B, k)).astype(np.int32)
    # 2 rows -> 16 splits of 4 blocks; entry 453 is in the third block of a split
    target = int(locs[0, 453])
    # K vector of the target row in float (fp8 latent * scale ; bf16 rope)
    row = dev[target].cpu()
    lat = row[:512].view(torch.float8_e4m3fn).float()
    sc = row[512:528].view(torch.float32)
    kvec = torch.cat([lat * sc.repeat_interleave(128), row[528:656].view(torch.bfloat16).float()])
    q = make_queries(B, H, seed=3, device="cuda").float().cpu()
    q[0, :4] = 8.0 * kvec / kvec.abs().max()       # heads 0..3 of row 0 point at the target
    q = q.to(torch.bfloat16).cuda().contiguous()
    got = _run_decode(dev, locs, q, H, k)
    ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                   dev.cpu().numpy(), float(np.float32(SCALE)))
    err = _normwise(got, ref)
    print("[decode] second pass max normwise error %.3g" % err.max(), flush=True)
    assert err.max() <= TOL


def test_decode_repeated_calls_on_one_pool():
    """Calls of different shapes on one pool: the split workspace grows, and
    a later call with fewer splits still reads only its own partials."""
    print("[decode] repeated calls", flush=True)
    rows = 1200
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 5, gen_device="cuda")
    hb = hs.HostBuffer(656 * 16)
    cfg = hs.PoolConfig(max_requests=1, slots=1024, max_top_k=1024, max_batch=8, max_seq_len=16,
                        max_heads=256)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], rows)
    try:
        for call, (B, H, k) in enumerate([(2, 128, 300), (7, 128, 1000), (2, 128, 300), (5, 256, 64),
                                          (7, 128, 1000)]):
            rng = np.random.default_rng(100 + call)
            locs = rng.integers(-1, rows, size=(B, k)).astype(np.int32)
            q = make_queries(B, H, seed=call, device="cuda")
            out = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
            hs.hisparse_sparse_mla_decode(pool, None, B, H, k, 0, q, torch.from_numpy(locs).cuda(),
                                          SCALE, out)
            torch.cuda.synchronize()
            got = out.float().cpu().numpy().astype(np.float64)
            ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                           dev.cpu().numpy(), float(np.float32(SCALE)))
            err = _normwise(got, ref)
            print("[decode] call %d B=%d H=%d k=%d max normwise error %.3g" % (call, B, H, k, err.max()),
                  flush=True)
            assert err.max() <= TOL
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


def test_decode_masked_keys_ignore_what_row_zero_holds():
    """Masked and out-of-range entries are read from row 0 and dequantised
    with a zero scale; with row 0 all 0xFF bytes (NaN latent codes, a NaN
    scale, NaN rope values) the output must still match the oracle, which
    skips those entries."""
    print("[decode] masked keys over a NaN row 0", flush=True)
    B, H, k, rows = 3, 64, 200, 700
    dev = torch.empty((rows, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 12, gen_device="cuda")
    dev[0].fill_(0xFF)
    rng = np.random.default_rng(12)
    locs = rng.integers(1, rows, size=(B, k)).astype(np.int32)
    locs[:, ::5] = -1
    locs[2, 1::9] = rows + 3
    q = make_queries(B, H, seed=12, device="cuda")
    got = _run_decode(dev, locs, q, H, k)
    assert np.all(np.isfinite(got))
    ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                   dev.cpu().numpy(), float(np.float32(SCALE)))
    err = _normwise(got, ref)
    print("[decode] masked keys max normwise error %.3g" % err.max(), flush=True)
    assert err.max() <= TOL


def test_decode_all_invalid_gives_zero():
    dev = torch.empty((64, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 3, gen_device="cuda")
    locs = np.full((2, 40), -1, np.int32)
    q = make_queries(2, 16, seed=1, device="cuda")
    got = _run_decode(dev, locs, q, 16, 40)
    assert np.all(got == 0)


def test_decode_zero_keys_writes_zeros():
    """top_k = 0: no entry to attend to, so every output is 0 (written over
    a NaN-filled buffer), through the pool and the allocation-free entry
    points."""
    B, H = 3, 144
    dev = torch.empty((64, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 5, gen_device="cuda")
    q = make_queries(B, H, seed=2, device="cuda")
    locs = torch.empty((B, 0), dtype=torch.int32, device="cuda")
    hb = hs.HostBuffer(656 * 16)
    cfg = hs.PoolConfig(max_requests=1, slots=16, max_top_k=16, max_batch=B, max_seq_len=16,
                        max_heads=H)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], dev.shape[0])
    try:
        for noalloc in (False, True):
            out = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            if noalloc:
                hs.hisparse_sparse_mla_decode_noalloc(None, B, H, 0, dev, q, locs, SCALE, out)
            else:
                hs.hisparse_sparse_mla_decode(pool, None, B, H, 0, 0, q, locs, SCALE, out)
            torch.cuda.synchronize()
            assert torch.equal(out.float(), torch.zeros((B, H, 512), device="cuda")), noalloc
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


def test_decode_after_resolver():
    """Resolver output feeds the decode on the same pool (small DSA-like)."""
    print("[decode+resolve]", flush=True)
    w = synth("dec", 41, R=6, S=512, k=256, steps=3, n0=[3000, 2500, 400, 8000, 100, 2000],
              grow=1, keep=200, recent=20, recent_window=256)
    bufs = make_host_pools(w, kind="mla")
    pair = Pair(w, bufs, max_heads=64)
    try:
        for step in range(w.steps):
            dst, src = pair.gpu_step(step)
            pair.oracle_step(step, dst, src)
        torch.cuda.synchronize()
        H = 64
        q = make_queries(w.B, H, seed=5, device="cuda")
        out = torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda")
        hs.hisparse_sparse_mla_decode(pair.pool, None, w.B, H, w.k, 0, q, pair.out, SCALE, out)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy().astype(np.float64)
        ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16),
                                       pair.out.cpu().numpy(), pair.ost.dev_pools[0],
                                       float(np.float32(SCALE)))
        err = _normwise(got, ref)
        print("[decode+resolve] max normwise error %.3g" % err.max(), flush=True)
        assert err.max() <= TOL
    finally:
        pair.close()


def _elementwise(got, ref, floor=1e-3):
    """Elementwise relative error with a floor on the denominator (reported
    for information; the normwise figure is the one with a tolerance)."""
    return (np.abs(got - ref) / np.maximum(np.abs(ref), floor)).max()


def _code_row(codes, scales):
    """One 656-byte row: 512 latent codes, four fp32 scales, zero rope."""
    row = np.zeros(656, np.uint8)
    row[:512] = codes
    row[512:528] = np.frombuffer(np.asarray(scales, np.float32).tobytes(), np.uint8)
    return row


def test_decode_every_e4m3_code_bit_exact():
    """Every OCP e4m3 code through the GPU's fp8 conversion: each batch row
    attends to one key (k = 1), so O is that row's V exactly, which is
    bf16(e4m3(code) * scale) and exact in bf16 for power-of-two scales.
    Rows 0 and 1 hold all 254 finite codes twice (in every scale block
    between them), with unit and with power-of-two scales down to the
    subnormal codes times 2^-7; the outputs must equal the oracle's float64
    values rounded to bf16, bit for bit.  Rows 2 and 3 hold the NaN codes
    0x7F and 0xFF: the oracle gives NaN for every output of such a row (its
    scores are NaN), and so must the kernel."""
    print("[decode] every e4m3 code", flush=True)
    codes = np.arange(512) % 256
    finite = np.where((codes & 0x7F) == 0x7F, 0, codes).astype(np.uint8)
    rolled = np.roll(finite, 128)
    rows_np = np.stack([
        _code_row(finite, [1.0, 1.0, 1.0, 1.0]),
        _code_row(rolled, [2.0 ** -7, 2.0 ** 5, 1.0, 2.0 ** -3]),
        _code_row(np.where(np.arange(512) == 5, 0x7F, finite), [1.0] * 4),
        _code_row(np.where(np.arange(512) == 300, 0xFF, rolled), [1.0, 0.5, 2.0, 1.0]),
    ] + [_code_row(finite, [1.0] * 4)] * 60)
    assert set(np.concatenate([rows_np[0, :512], rows_np[1, :512]]).tolist()) == \
        set(range(256)) - {0x7F, 0xFF}
    dev = torch.from_numpy(rows_np).cuda()
    B, H = 4, 16
    locs = np.arange(B, dtype=np.int32).reshape(B, 1)
    q = make_queries(B, H, seed=256, device="cuda")
    got_t = torch.from_numpy(_run_decode(dev, locs, q, H, 1)).to(torch.bfloat16)
    ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                   rows_np, float(np.float32(SCALE)))
    ref_t = torch.from_numpy(ref).to(torch.bfloat16)
    for b in (0, 1):
        assert torch.equal(got_t[b].view(torch.int16), ref_t[b].view(torch.int16)), \
            "row %d: %d outputs differ" % (b, int((got_t[b] != ref_t[b]).sum()))
        # and the oracle's value is the OCP decode times the scale
        lat = torch.from_numpy(rows_np[b, :512].copy()).view(torch.float8_e4m3fn).double()
        sc = torch.from_numpy(rows_np[b, 512:528].copy()).view(torch.float32).double()
        assert torch.equal(torch.from_numpy(ref[b, 0]), lat * sc.repeat_interleave(128))
    for b in (2, 3):
        assert np.isnan(ref[b]).all()
        assert torch.isnan(got_t[b].float()).all(), "row %d: a NaN code must give NaN" % b
    print("[decode] 254 finite codes bit-exact, NaN codes give NaN", flush=True)


def test_config5_full_size_every_row():
    """Config 5: the DSA-decode resolver output (72 rows: 64 long rows of
    top-2048 and 8 fast-path rows) feeds 128-head decode; every batch row and
    every head is compared with the float64 oracle."""
    print("[config5] generating", flush=True)
    w = config2_dsa_decode(steps=4)
    bufs = make_host_pools(w, kind="mla")
    pair = Pair(w, bufs, with_oracle=False, max_heads=128)
    try:
        for step in range(w.steps):
            pair.gpu_step(step)
        torch.cuda.synchronize()
        H = 128
        q = make_queries(w.B, H, seed=55, device="cuda")
        out = torch.empty((w.B, H, 512), dtype=torch.bfloat16, device="cuda")
        hs.hisparse_sparse_mla_decode(pair.pool, None, w.B, H, w.k, 0, q, pair.out, SCALE, out)
        torch.cuda.synchronize()
        locs = pair.out.cpu().numpy()
        assert (locs >= 0).sum() == (w.top_k[w.steps - 1] >= 0).sum()
        print("[config5] oracle on all %d batch rows x %d heads" % (w.B, H), flush=True)
        ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16), locs,
                                       pair.dev_pools[0].cpu().numpy(), float(np.float32(SCALE)))
        got = out.float().cpu().numpy().astype(np.float64)
        err = _normwise(got, ref)
        print("[config5] max normwise error %.4g over %d (row, head) pairs; elementwise with a "
              "1e-3 floor %.4g" % (err.max(), err.size, _elementwise(got, ref)), flush=True)
        assert err.shape == (w.B, H)
        assert err.max() <= TOL
    finally:
        pair.close()
