"""Test harness: runs one workload step by step on the HIP library and on the
CPU oracle from the same inputs and compares everything.

Set-up only (allocation, admission copies, uploads); no step of the method
is computed here.
"""
from __future__ import annotations

import numpy as np
import torch

import hierarchical_sparse_attention_hisparse_amd as hs
from oracle import OracleState, oracle_resolve
from workloads import admission, decode_writes, fill_host_rows_uniform, fill_host_rows_mla


def make_host_pools(w, kind="uniform", seed_base=100, gen_device="cuda"):
    """One pinned HostBuffer per layer, filled with seeded row bytes."""
    bufs = []
    for l in range(w.L):
        hb = hs.HostBuffer(max(16, w.host_pool_rows * w.row_bytes))
        t = hb.torch((w.host_pool_rows, w.row_bytes))
        if kind == "uniform":
            fill_host_rows_uniform(t, seed_base + l, gen_device=gen_device)
        else:
            fill_host_rows_mla(t, seed_base + l, gen_device=gen_device)
        bufs.append(hb)
    return bufs


class Pair:
    """The GPU side and the oracle side of one workload."""

    def __init__(self, w, host_bufs, with_oracle=True, max_batch=None, mode="resolve",
                 max_steps=1, max_heads=0):
        """mode "resolve": the single-call entry point (which copies inside the
        plan kernel at batch >= 8 with <= 8 layers); "split": the plan entry
        point followed by the separate copy entry point.  max_heads > 0 gives
        the pool a decode workspace for up to that many heads."""
        assert mode in ("resolve", "split")
        self.mode = mode
        self.w = w
        self.host_bufs = host_bufs
        self.host_np = [h.numpy((w.host_pool_rows, w.row_bytes)) for h in host_bufs]
        self.host_t = [torch.from_numpy(a) for a in self.host_np]
        dev = torch.device("cuda")
        self.dev_pools = [torch.zeros((w.dev_pool_rows, w.row_bytes), dtype=torch.uint8, device=dev)
                          for _ in range(w.L)]
        cfg = hs.PoolConfig(max_requests=w.R, slots=w.S, max_top_k=w.k,
                            max_batch=max_batch or w.B, row_bytes=w.row_bytes,
                            num_layers=w.L, page_size=w.P, resident_pages=w.resident_pages,
                            max_seq_len=w.max_seq_len, max_steps=max_steps,
                            max_heads=max_heads)
        self.pool = hs.hisparse_init_pool(cfg, host_bufs, [w.host_pool_rows] * w.L,
                                          self.dev_pools, w.dev_pool_rows)
        st, lru, clk, dst, src = admission(w)
        self.st = torch.from_numpy(st).to(dev)
        self.lru = torch.from_numpy(lru).to(dev)
        self.clk = torch.from_numpy(clk).to(dev)
        self.stats = torch.zeros(5, dtype=torch.int64, device=dev)
        self.req_idx = torch.from_numpy(w.req_idx).to(dev)
        self.locs = torch.from_numpy(w.host_cache_locs).to(dev)
        self.bt = torch.from_numpy(w.block_table).to(dev) if w.block_table is not None else None
        self.topk = torch.from_numpy(w.top_k).to(dev)
        self.seq = torch.from_numpy(w.seq_lens).to(dev)
        self.out = torch.empty((w.B, w.k), dtype=torch.int32, device=dev)
        self._copy_rows(dst, src)
        self.ost = None
        if with_oracle:
            self.ost = OracleState(R=w.R, S=w.S, L=w.L, row_bytes=w.row_bytes,
                                   dev_pool_rows=w.dev_pool_rows)
            self.ost.slot_tokens[:], self.ost.lru_slots[:], self.ost.lru_clock[:] = st, lru, clk
            for l in range(w.L):
                if len(dst):
                    self.ost.dev_pools[l][dst] = self.host_np[l][src]
        torch.cuda.synchronize()

    def _copy_rows(self, dst, src):
        if len(dst) == 0:
            return
        d = torch.from_numpy(dst).cuda()
        for l in range(self.w.L):
            rows = self.host_t[l][torch.from_numpy(src)].cuda()
            self.dev_pools[l].index_copy_(0, d, rows)

    def writes_of(self, step):
        """The forward pass's fast-path row writes before `step`."""
        return decode_writes(self.w, step)

    def pre_step_writes(self, step):
        """Apply those writes to the GPU pools only (the oracle applies them in
        oracle_step)."""
        dst, src = decode_writes(self.w, step)
        self._copy_rows(dst, src)
        return dst, src

    def gpu_step(self, step, stream=None):
        w = self.w
        dst, src = decode_writes(w, step)
        self._copy_rows(dst, src)
        args = (self.pool, stream, w.B, w.k, self.req_idx, self.topk[step], self.seq[step],
                self.locs, self.bt, self.st, self.lru, self.clk, self.out, self.stats)
        if self.mode == "resolve":
            hs.hisparse_resolve(*args)
        else:
            hs.hisparse_resolve_plan(*args)
            hs.hisparse_gather_copy(self.pool, stream, w.B, 0, w.L, self.stats)
        return dst, src

    def oracle_step(self, step, dst, src):
        w = self.w
        for l in range(w.L):
            if len(dst):
                self.ost.dev_pools[l][dst] = self.host_np[l][src]
        return oracle_resolve(self.ost, page_size=w.P, max_seq_len=w.max_seq_len,
                              resident_pages=w.resident_pages, req_idx=w.req_idx,
                              top_k_tokens=w.top_k[step], seq_lens=w.seq_lens[step],
                              host_cache_locs=w.host_cache_locs, block_table=w.block_table,
                              host_pools=self.host_np, host_pool_rows=[w.host_pool_rows] * w.L)

    def compare_step(self, step, o_out, check_rows=True):
        w = self.w
        g_out = self.out.cpu().numpy()
        assert np.array_equal(g_out, o_out), _first_diff("device_buffer_locs", g_out, o_out)
        for name, g, o in (("slot_tokens", self.st, self.ost.slot_tokens),
                           ("lru_slots", self.lru, self.ost.lru_slots),
                           ("lru_clock", self.clk, self.ost.lru_clock)):
            ga = g.cpu().numpy()
            assert np.array_equal(ga, o), _first_diff(name, ga, o)
        gs = self.stats.cpu().numpy().astype(np.uint64)
        assert np.array_equal(gs, self.ost.stats), ("stats", gs, self.ost.stats)
        if check_rows:
            rows = np.unique(o_out[o_out >= 0])
            if len(rows):
                ridx = torch.from_numpy(rows.astype(np.int64)).cuda()
                for l in range(w.L):
                    g = self.dev_pools[l].index_select(0, ridx).cpu().numpy()
                    o = self.ost.dev_pools[l][rows]
                    assert np.array_equal(g, o), _first_diff("rows of layer %d" % l, g, o)

    def compare_pools(self):
        for l in range(self.w.L):
            g = self.dev_pools[l].cpu().numpy()
            assert np.array_equal(g, self.ost.dev_pools[l]), _first_diff(
                "device pool %d" % l, g, self.ost.dev_pools[l])

    def close(self):
        hs.hisparse_destroy_pool(self.pool)


def _first_diff(name, g, o):
    bad = np.argwhere(g != o)
    if len(bad) == 0:
        return name + ": shapes differ %s vs %s" % (g.shape, o.shape)
    i = tuple(bad[0])
    return "%s differs at %d places, first at %s: gpu=%s oracle=%s" % (name, len(bad), i, g[i], o[i])


def run_parity(w, steps=None, kind="uniform", check_rows=True, host_bufs=None, log=None,
               mode="resolve"):
    """Run `steps` steps of workload w on both sides, comparing every step."""
    steps = w.steps if steps is None else steps
    bufs = host_bufs or make_host_pools(w, kind)
    pair = Pair(w, bufs, mode=mode)
    try:
        for step in range(steps):
            dst, src = pair.gpu_step(step)
            o_out = pair.oracle_step(step, dst, src)
            torch.cuda.synchronize()
            pair.compare_step(step, o_out, check_rows=check_rows)
            if log:
                log(step)
        pair.compare_pools()
        return pair.ost.stats.copy()
    finally:
        pair.close()
