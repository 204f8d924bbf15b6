"""An independent, deliberately different formulation of the resolver rules,
used only to pin the C oracle on tiny inputs.

Where the oracle sorts all candidate slots once, this one looks hits up in a
dict and, for every miss in turn, scans every slot for the smallest key
(occupied, stamp, slot) among those neither hit nor already handed out.
Rules restated from "vLLM HiSparse 本地 KV 卸载架构" (hot-row lookup and LRU)
and "vLLM Hybrid HiSparse 源码实现分析" sections 7.2-7.4.
"""
import numpy as np


def _wrap32(x):
    return int(np.int32(np.uint32((int(x) + (1 << 32)) % (1 << 32))))


def naive_resolve(st, lru, clk, stats, dev_pools, *, R, S, P, max_seq_len,
                  resident_pages, req_idx, topk, seq_lens, locs, bt,
                  host_pools, host_rows, row_bytes):
    B, k = topk.shape
    out = np.full((B, k), -1, dtype=np.int32)
    for b in range(B):
        r = int(req_idx[b])
        if r < 0 or r >= R:
            if r >= R:
                stats[4] += 1
            continue
        n = min(int(seq_lens[b]), max_seq_len)
        c = _wrap32(int(clk[r]) + 1)
        clk[r] = c
        row = [int(x) for x in topk[b]]
        if int(seq_lens[b]) <= S:
            for i, t in enumerate(row):
                if 0 <= t < n:
                    out[b, i] = r * S + t
                    st[r, t] = t
                    lru[r, t] = c
                    stats[3] += 1
            continue
        pending = []
        for i, t in enumerate(row):
            if not (0 <= t < n):
                continue
            if bt is not None and P > 0:
                p = int(bt[r, t // P])
                if 0 <= p < resident_pages:
                    out[b, i] = R * S + p * P + t % P
                    stats[2] += 1
                    continue
                if p >= 0:
                    stats[4] += 1
            pending.append((i, t))
        where = {}
        for s in range(S):
            tok = int(st[r, s])
            if tok >= 0 and tok not in where:
                where[tok] = s
        keys = {s: (1 if int(st[r, s]) >= 0 else 0, int(lru[r, s]), s) for s in range(S)}
        hit_slots = set()
        misses = []
        for i, t in pending:
            if t in where:
                s = where[t]
                out[b, i] = r * S + s
                lru[r, s] = c
                hit_slots.add(s)
                stats[0] += 1
            else:
                misses.append((i, t))
        taken = set()
        for i, t in misses:
            best = None
            for s in range(S):
                if s in hit_slots or s in taken:
                    continue
                if best is None or keys[s] < keys[best]:
                    best = s
            taken.add(best)
            st[r, best] = t
            lru[r, best] = c
            out[b, i] = r * S + best
            h = int(locs[r, t])
            for l in range(len(dev_pools)):
                if 0 <= h < host_rows[l]:
                    dev_pools[l][r * S + best] = host_pools[l][h]
                else:
                    dev_pools[l][r * S + best] = 0
                    stats[4] += 1
            stats[1] += 1
    return out
