"""Seeded synthetic workloads for the HiSparse swap-in resolver.

Inputs only: no step of the resolver or of attention is computed here.  The
shapes and mixes stand in for the decode workloads the pages describe (DSA
top-2048 selection, hot buffers of 2-3x top-k, adjacent-step top-k overlap
of 80-90 % as in "分层稀疏注意力框架下的 KV 分层管理与按需加载", section 2.4.3;
1M-token GLM contexts with index-shared layers as in "vLLM Hybrid HiSparse
源码实现分析", section 7.4).  The traces the pages measured on (LongBenchV2,
OpenHands) are not available; these seeded generators replace them.

Random numbers come from numpy's PCG64 (top-k traces, placement, block
tables) and torch's generator (row bytes, queries), all seeded per workload.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

ROW_BYTES = 656          # 512 B fp8 latent + 16 B fp32 scales + 128 B bf16 rope
HOST_PAGE = 64           # host rows are placed in pages of 64 tokens


@dataclass
class Workload:
    name: str
    R: int                      # request-state rows
    S: int                      # hot slots per request (device_buffer_size)
    k: int                      # top-k width
    L: int                      # layers sharing one plan
    P: int                      # resident page size (0: no resident tier)
    B: int                      # batch rows
    steps: int
    max_seq_len: int            # row stride of host_cache_locs (tokens)
    req_idx: np.ndarray         # [B] int32
    seq_lens: np.ndarray        # [steps, B] int32
    top_k: np.ndarray           # [steps, B, k] int32, -1 = padding entry
    host_cache_locs: np.ndarray  # [R, max_seq_len] int64 host row per token
    host_pool_rows: int         # rows of each layer's host pool
    resident_pages: int = 0
    block_table: Optional[np.ndarray] = None  # [R, max_pages] int32, -1 = host
    seed: int = 0
    row_bytes: int = ROW_BYTES
    meta: dict = field(default_factory=dict)
    extra_dev_rows: int = 0     # device rows after the hot and resident rows (staging)

    @property
    def dev_pool_rows(self) -> int:
        return self.R * self.S + self.resident_pages * self.P + self.extra_dev_rows

    @property
    def max_pages(self) -> int:
        return (self.max_seq_len + self.P - 1) // self.P if self.P > 0 else 0

    def valid_entries(self, step: int) -> int:
        """Number of top-k entries of `step` inside [0, seq_len) on active rows."""
        tk = self.top_k[step]
        n = self.seq_lens[step][:, None]
        act = (self.req_idx >= 0)[:, None]
        return int(((tk >= 0) & (tk < n) & act).sum())


# --------------------------------------------------------------------------
# top-k traces
# --------------------------------------------------------------------------

def _draw_distinct(rng, lo, hi, count, mask, out):
    """Append `count` distinct positions uniform on [lo, hi) that are not yet
    marked in `mask` (rejection sampling), marking them."""
    hi = max(lo, hi)
    avail = (hi - lo) - int(mask[lo:hi].sum()) if hi > lo else 0
    count = min(count, avail)
    while count > 0:
        cand = rng.integers(lo, hi, size=max(2 * count, 16))
        _, first = np.unique(cand, return_index=True)
        cand = cand[np.sort(first)]
        cand = cand[~mask[cand]][:count]
        mask[cand] = True
        out.append(cand)
        count -= len(cand)


def _zipf_cdf(nblocks: int, s: float) -> np.ndarray:
    w = np.arange(1, nblocks + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def _row_topk(rng, prev, n, k, spec, zipf_perm=None, zipf_cdf=None):
    """One row of top-k positions for sequence length n (distinct, shuffled)."""
    if n <= k:
        row = np.full(k, -1, dtype=np.int64)
        row[:n] = np.arange(n)
        return rng.permutation(row).astype(np.int32)
    mask = np.zeros(n, dtype=bool)
    parts = []
    if prev is not None and spec["keep"] > 0:
        p = prev[(prev >= 0) & (prev < n)]
        keep = rng.choice(p, size=min(spec["keep"], len(p)), replace=False)
        mask[keep] = True
        parts.append(keep)
    if spec.get("recent_all", 0) > 0:
        ra = np.arange(max(0, n - spec["recent_all"]), n)
        ra = ra[~mask[ra]]
        mask[ra] = True
        parts.append(ra)
    if spec.get("blocks", 0) > 0:
        bs = spec["block_size"]
        nb = (n - spec.get("recent_all", 0)) // bs
        got = 0
        while got < spec["blocks"]:
            u = rng.random()
            rank = int(np.searchsorted(zipf_cdf, u, side="right"))
            rank = min(rank, nb - 1)
            blk = int(zipf_perm[rank])
            toks = np.arange(blk * bs, blk * bs + bs)
            if mask[toks].any():
                continue            # duplicate block: rejected
            mask[toks] = True
            parts.append(toks)
            got += 1
    if spec.get("recent", 0) > 0:
        _draw_distinct(rng, n - spec["recent_window"], n, spec["recent"], mask, parts)
    have = sum(len(x) for x in parts)
    _draw_distinct(rng, 0, n, k - have, mask, parts)
    row = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    assert len(row) == k, (len(row), k)
    return rng.permutation(row).astype(np.int32)


def _placement(rng, R, n_final, max_seq_len):
    """host_cache_locs: each request's tokens live in host pages of 64 rows,
    the pages of all requests scattered by one seeded permutation."""
    pages = (np.asarray(n_final, dtype=np.int64) + HOST_PAGE - 1) // HOST_PAGE
    total = int(pages.sum())
    perm = rng.permutation(total).astype(np.int64)
    locs = np.full((R, max_seq_len), -1, dtype=np.int64)
    off = 0
    for r in range(R):
        npg = int(pages[r])
        t = np.arange(npg * HOST_PAGE, dtype=np.int64)
        t = t[t < max_seq_len]
        locs[r, :len(t)] = perm[off + t // HOST_PAGE] * HOST_PAGE + t % HOST_PAGE
        off += npg
    return locs, total * HOST_PAGE


def synth(name, seed, *, R, S, k, steps, n0, L=1, grow=0, keep=0, recent=0,
          recent_window=0, recent_all=0, blocks=0, block_size=32, zipf_s=1.1,
          P=0, resident_tail=0, req_perm=True, padding_rows=0) -> Workload:
    """General seeded workload.

    n0: initial seq_len per batch row (array of B values); grow: tokens added
    per step.  Per step and row: `keep` positions kept from the previous step,
    all of the last `recent_all` positions, `blocks` Zipf-drawn blocks of
    `block_size` tokens, `recent` positions from the last `recent_window`, and
    uniform positions for the rest.  Step 0 has no kept part.  Rows with
    seq_len <= k take all of [0, seq_len) padded with -1.  `padding_rows`
    batch rows get req_idx = -1.  With P > 0 and resident_tail > 0 the last
    `resident_tail` tokens of every request sit in resident pages mapped by a
    seeded permutation.
    """
    rng = np.random.default_rng(seed)
    n0 = np.asarray(n0, dtype=np.int64)
    nb_active = len(n0)
    B = nb_active + padding_rows
    assert nb_active <= R
    active_req = rng.permutation(R)[:nb_active] if req_perm else np.arange(nb_active)
    req_unshuffled = np.concatenate([active_req, np.full(padding_rows, -1)]).astype(np.int64)
    n0_unshuffled = np.concatenate([n0, np.zeros(padding_rows, dtype=np.int64)])
    order = rng.permutation(B) if req_perm else np.arange(B)
    req_idx = req_unshuffled[order].astype(np.int32)
    n0_rows = n0_unshuffled[order]
    # sequence lengths per step
    seq = n0_rows[None, :] + grow * np.arange(steps, dtype=np.int64)[:, None]
    seq[:, req_idx < 0] = 0
    n_final_req = np.zeros(R, dtype=np.int64)
    for b in range(B):
        if req_idx[b] >= 0:
            n_final_req[req_idx[b]] = seq[-1, b]
    max_seq_len = int(((n_final_req.max() + HOST_PAGE - 1) // HOST_PAGE) * HOST_PAGE)
    if P > 0:
        max_seq_len = int(((max_seq_len + P - 1) // P) * P)
    locs, host_rows = _placement(rng, R, n_final_req, max_seq_len)

    spec = dict(keep=keep, recent=recent, recent_window=recent_window,
                recent_all=recent_all, blocks=blocks, block_size=block_size)
    zipf_cdf = None
    top = np.full((steps, B, k), -1, dtype=np.int32)
    for b in range(B):
        if req_idx[b] < 0:
            continue
        prev = None
        zipf_perm = None
        for st in range(steps):
            n = int(seq[st, b])
            if blocks > 0:
                nb = (n - recent_all) // block_size
                if zipf_cdf is None or len(zipf_cdf) != nb:
                    zipf_cdf = _zipf_cdf(nb, zipf_s)
                if zipf_perm is None or len(zipf_perm) != nb:
                    zipf_perm = rng.permutation(nb)     # rank -> block, per request
            sp = dict(spec)
            if prev is None:
                sp["keep"] = 0
            row = _row_topk(rng, prev, n, k, sp, zipf_perm, zipf_cdf)
            top[st, b] = row
            prev = row.astype(np.int64)

    block_table = None
    resident_pages = 0
    if P > 0 and resident_tail > 0:
        max_pages = max_seq_len // P
        block_table = np.full((R, max_pages), -1, dtype=np.int32)
        tail_pages = resident_tail // P
        resident_pages = R * tail_pages
        phys = rng.permutation(resident_pages).astype(np.int32)
        for r in range(R):
            n_r = int(n_final_req[r])
            first = n_r // P - tail_pages
            if n_r == 0 or first < 0:
                continue                # inactive or too short: no resident tail
            block_table[r, first:first + tail_pages] = phys[r * tail_pages:(r + 1) * tail_pages]

    return Workload(name=name, R=R, S=S, k=k, L=L, P=P, B=B, steps=steps,
                    max_seq_len=max_seq_len, req_idx=req_idx,
                    seq_lens=seq.astype(np.int32), top_k=top,
                    host_cache_locs=locs, host_pool_rows=host_rows,
                    resident_pages=resident_pages, block_table=block_table,
                    seed=seed)


# --------------------------------------------------------------------------
# the five named configurations
# --------------------------------------------------------------------------

def config1_tiny(seed=1, steps=32) -> Workload:
    """4 requests of 8192 tokens, top-256, 512 slots, 80 % kept, 20 % uniform."""
    return synth("tiny", seed, R=4, S=512, k=256, steps=steps, n0=[8192] * 4,
                 keep=204)


def config2_dsa_decode(seed=2, steps=64, long_rows=64, short_rows=8) -> Workload:
    """64 long rows (seq_len U[32768, 131072]) + 8 short fast-path rows
    (seq_len U[1024, 4032]); top-2048, 4096 slots, seq_len +1 per step;
    90 % kept, 5 % from the last 2048 positions, 5 % uniform."""
    rng = np.random.default_rng(seed + 1000)
    n_long = rng.integers(32768, 131072 + 1, size=long_rows)
    n_short = rng.integers(1024, 4032 + 1, size=short_rows)
    n0 = np.concatenate([n_long, n_short])
    return synth("dsa_decode", seed, R=long_rows + short_rows, S=4096, k=2048,
                 steps=steps, n0=n0, grow=1, keep=1843, recent=102,
                 recent_window=2048)


def config3_mixed_residency(f=0.9, seed=3, steps=32, R=128, n=131072) -> Workload:
    """128 requests of 131072 tokens whose last 16384 tokens sit in resident
    pages of 64; 4096 slots, top-2048 with floor(f*k) kept, rest uniform."""
    k = 2048
    w = synth("mixed_residency_f%g" % f, seed, R=R, S=4096, k=k, steps=steps,
              n0=[n] * R, keep=int(math.floor(f * k)), P=64, resident_tail=16384)
    w.meta["reuse"] = f
    return w


def config4_indexshare_1m(seed=4, steps=32, R=16, n=1048576) -> Workload:
    """16 requests of 1M tokens, 6144 slots, 4 layers sharing one plan;
    per step the last 512 positions plus 48 Zipf(1.1)-drawn 32-token blocks."""
    return synth("indexshare_1m", seed, R=R, S=6144, k=2048, steps=steps,
                 n0=[n] * R, L=4, recent_all=512, blocks=48, block_size=32,
                 zipf_s=1.1)


# --------------------------------------------------------------------------
# admission and decode-time KV writes (harness set-up, identical for both
# sides of a comparison)
# --------------------------------------------------------------------------

def admission(w: Workload):
    """Initial resolver state and the device rows to fill before step 0.

    Requests whose first seq_len fits the hot buffer start on the fast path:
    slot t holds token t (stamp 0) and its device row holds the token's host
    row.  Longer requests start with every slot empty (rows are loaded only
    when selected).  Resident pages hold their tokens' host rows.
    Returns (slot_tokens, lru_slots, lru_clock, dst_rows, src_host_rows).
    """
    st = np.full((w.R, w.S), -1, dtype=np.int32)
    lru = np.zeros((w.R, w.S), dtype=np.int32)
    clk = np.zeros((w.R,), dtype=np.int32)
    dst, src = [], []
    for b in range(w.B):
        r = int(w.req_idx[b])
        if r < 0 or r >= w.R:
            continue
        n0 = int(w.seq_lens[0, b])
        if n0 <= w.S:
            t = np.arange(n0)
            st[r, :n0] = t
            dst.append(r * w.S + t)
            src.append(w.host_cache_locs[r, :n0])
    if w.block_table is not None:
        for r in range(w.R):
            pages = np.nonzero(w.block_table[r] >= 0)[0]
            for j in pages:
                p = int(w.block_table[r, j])
                o = np.arange(w.P)
                dst.append(w.R * w.S + p * w.P + o)
                src.append(w.host_cache_locs[r, j * w.P + o])
    dst = np.concatenate(dst).astype(np.int64) if dst else np.zeros(0, np.int64)
    src = np.concatenate(src).astype(np.int64) if src else np.zeros(0, np.int64)
    return st, lru, clk, dst, src


def decode_writes(w: Workload, step: int):
    """Rows the forward pass writes before `step` on fast-path requests: the
    tokens appended since the previous step go to slot == position."""
    dst, src = [], []
    if step == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    for b in range(w.B):
        r = int(w.req_idx[b])
        if r < 0 or r >= w.R:
            continue
        n_prev, n = int(w.seq_lens[step - 1, b]), int(w.seq_lens[step, b])
        if n <= w.S and n > n_prev:
            t = np.arange(n_prev, n)
            dst.append(r * w.S + t)
            src.append(w.host_cache_locs[r, t])
    if not dst:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return np.concatenate(dst).astype(np.int64), np.concatenate(src).astype(np.int64)


# --------------------------------------------------------------------------
# row bytes and queries (torch generators, chunked)
# --------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def fill_host_rows_uniform(dst, seed: int, gen_device: str = "cpu",
                           chunk_rows: int = 1 << 20):
    """Fill a [rows, 656] uint8 host tensor with seeded uniform random bytes."""
    torch = _torch()
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    rows = dst.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randint(0, 256, (r1 - r0, dst.shape[1]), dtype=torch.uint8,
                          generator=g, device=gen_device)
        dst[r0:r1].copy_(x)


def fill_host_rows_mla(dst, seed: int, gen_device: str = "cpu",
                       chunk_rows: int = 1 << 18):
    """Fill [rows, 656] uint8 with sparse-MLA rows: a N(0,1) latent of 512
    values stored as fp8 e4m3 with one fp32 scale per 128 values
    (scale = amax / 448, 1 when amax = 0), then 64 N(0,1) rope values in
    bf16.  The quantisation is done by torch's own fp8/bf16 casts."""
    torch = _torch()
    g = torch.Generator(device=gen_device)
    g.manual_seed(seed)
    rows = dst.shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        m = r1 - r0
        lat = torch.randn((m, 4, 128), generator=g, device=gen_device, dtype=torch.float32)
        amax = lat.abs().amax(dim=2, keepdim=True)
        scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
        q8 = (lat / scale).to(torch.float8_e4m3fn)
        rope = torch.randn((m, 64), generator=g, device=gen_device,
                           dtype=torch.float32).to(torch.bfloat16)
        out = torch.cat([q8.reshape(m, 512).view(torch.uint8),
                         scale.reshape(m, 4).contiguous().view(torch.uint8),
                         rope.view(torch.uint8)], dim=1)
        dst[r0:r1].copy_(out)


def make_queries(B: int, H: int, seed: int, device: str = "cpu"):
    """bf16 queries [B, H, 576] drawn N(0,1) (512 latent + 64 rope dims)."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn((B, H, 576), generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)
