"""The allocation-free decode entry point (hisparse_sparse_mla_decode_noalloc)
called through the C ABI: its output equals the pool entry point's
(hisparse_sparse_mla_decode) bit for bit on the same rows, over calls in a
row on the shared static workspace, each smaller than the one before; the
smallest is also checked against the float64 oracle.  Shapes beyond the
static workspace are refused on the host."""
import ctypes
import math

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from oracle import oracle_sparse_mla_decode
from workloads import fill_host_rows_mla, make_queries

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(192.0)
ROWS = 4096


def _noalloc(lib, dev, B, H, k, q, locs, out):
    return lib.hisparse_sparse_mla_decode_noalloc(
        None, B, H, k, ctypes.c_void_p(dev.data_ptr()), ctypes.c_int64(dev.shape[0]),
        dev.shape[1], ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(locs.data_ptr()),
        ctypes.c_float(SCALE), ctypes.c_void_p(out.data_ptr()))


def test_noalloc_decode_equals_the_pool_entry_point():
    lib = hs.load_library()
    dev = torch.empty((ROWS, 656), dtype=torch.uint8, device="cuda")
    fill_host_rows_mla(dev, 404, gen_device="cuda")
    hb = hs.HostBuffer(656 * 16)
    cfg = hs.PoolConfig(max_requests=1, slots=2048, max_top_k=2048, max_batch=256, max_seq_len=16,
                        max_heads=128)
    pool = hs.hisparse_init_pool(cfg, [hb], [16], [dev], ROWS)
    try:
        # the largest call the static workspace holds (256 rows x 1 head
        # group x 1 split), then two smaller ones (240 units of 6 splits;
        # 48 units of 16 splits)
        for call, (B, H, k) in enumerate([(256, 128, 96), (40, 128, 2048), (3, 64, 500)]):
            print("[noalloc] call %d: B=%d H=%d k=%d" % (call, B, H, k), flush=True)
            rng = np.random.default_rng(40 + call)
            locs_np = rng.integers(0, ROWS, size=(B, k)).astype(np.int32)
            locs_np[rng.random((B, k)) < 0.1] = -1
            locs_np[0, -1] = ROWS + 3          # out of range: skipped
            locs = torch.from_numpy(locs_np).cuda()
            q = make_queries(B, H, seed=410 + call, device="cuda")
            want = torch.empty((B, H, 512), dtype=torch.bfloat16, device="cuda")
            hs.hisparse_sparse_mla_decode(pool, None, B, H, k, 0, q, locs, SCALE, want)
            got = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            rc = _noalloc(lib, dev, B, H, k, q, locs, got)
            assert rc == 0, hs.hisparse_last_error()
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), \
                "call %d: %d outputs differ" % (call, int((got != want).sum()))
            if B <= 4:
                ref = oracle_sparse_mla_decode(q.cpu().view(torch.int16).numpy().astype(np.uint16),
                                               locs_np, dev.cpu().numpy(), float(np.float32(SCALE)))
                g = got.float().cpu().numpy().astype(np.float64)
                err = np.abs(g - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)
                print("[noalloc] call %d: max normwise error vs the oracle %.3g" % (call, err.max()),
                      flush=True)
                assert err.max() <= 2e-2
        # the binding's wrapper of the same entry point
        out = torch.empty((3, 64, 512), dtype=torch.bfloat16, device="cuda")
        hs.hisparse_sparse_mla_decode_noalloc(None, 3, 64, 500, dev, q, locs, SCALE, out)
        torch.cuda.synchronize()
        assert torch.equal(out, got)
    finally:
        hs.hisparse_destroy_pool(pool)
        hb.free()


def test_noalloc_decode_refuses_what_the_static_workspace_cannot_hold():
    """Refusals happen on the host before anything is enqueued."""
    lib = hs.load_library()
    dev = torch.zeros((64, 656), dtype=torch.uint8, device="cuda")
    q = torch.zeros((257, 128, 576), dtype=torch.bfloat16, device="cuda")
    locs = torch.zeros((257, 8), dtype=torch.int32, device="cuda")
    out = torch.zeros((257, 128, 512), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(lib, dev, 257, 128, 8, q, locs, out) == -4
    assert "256" in hs.hisparse_last_error()
    assert _noalloc(lib, dev, 129, 256, 8, q, locs, out) == -4      # 2 head groups x 129 rows
    assert _noalloc(lib, dev, 2, 20, 8, q, locs, out) == -4         # heads not a multiple of 16
    assert _noalloc(lib, dev, 2, 16, 5000, q, locs, out) == -1      # top_k beyond 4096
    small = torch.zeros((64, 640), dtype=torch.uint8, device="cuda")
    assert _noalloc(lib, small, 2, 16, 8, q, locs, out) == -4       # rows too short
    torch.cuda.synchronize()
    assert int(out.abs().sum().item()) == 0                        # nothing ran
