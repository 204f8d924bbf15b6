// resolve.hip -- the resolver's plan kernel for gfx950.
//
// One workgroup of 1024 threads (16 wavefronts) per batch row.  For one
// request it performs, in LDS:
//   1. validity + resident short-circuit, then hashing of the remaining
//      positions into an open-addressing table (position -> top-k index);
//   2. one pass over the request's S slots (slot_tokens and stamps staged in
//      LDS) that probes the table: a slot holding a wanted position is a hit;
//   3. hit row IDs and stamp refreshes, and a block-wide exclusive scan that
//      lists the misses in ascending top-k index;
//   4. victim ranking over the non-hit slots by the key (occupied, stamp,
//      slot): repeated block-wide minimum extraction with a stable (slot
//      order) prefix-sum rank inside each key value, and a bitonic sort of
//      the remaining candidates if a few rounds do not cover all misses;
//   5. the j-th miss takes the j-th victim: new token, stamp, row ID, and one
//      (host row, device row) entry of the compact miss plan.
// The resolution order and phases follow "vLLM HiSparse 本地 KV 卸载架构"
// (hot-row lookup and LRU) and "vLLM Hybrid HiSparse 源码实现分析" section
// 7.2; the fast path (seq_len <= S: slot == position, nothing moves) follows
// the per-step flow of the gogongxt.com HiSparse page.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

__device__ inline int block_exscan(int v, int* s_wave, int* total) {
  const int ln = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(x, d, kWave);
    if (ln >= d) x += y;
  }
  if (ln == kWave - 1) s_wave[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kResolveWaves; ++i) {
    const int t = s_wave[i];
    base += (i < w) ? t : 0;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ inline uint64_t block_min_u64(uint64_t v, uint64_t* s_red) {
  const int ln = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) {
    const uint64_t o = __shfl_xor(v, d, kWave);
    v = o < v ? o : v;
  }
  if (ln == 0) s_red[w] = v;
  __syncthreads();
  uint64_t m = s_red[0];
#pragma unroll
  for (int i = 1; i < kResolveWaves; ++i) {
    const uint64_t t = s_red[i];
    m = t < m ? t : m;
  }
  __syncthreads();
  return m;
}

__device__ inline int wave_sum(int v) {
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

// Victim key of a slot without its slot index: (occupied, stamp) with the
// signed stamp mapped to an order-preserving unsigned value.
__device__ inline uint64_t key33(const int32_t* s_tok, const int32_t* s_stamp, int s) {
  const uint64_t occ = s_tok[s] >= 0 ? 1ull : 0ull;
  return (occ << 32) | (uint64_t)((uint32_t)s_stamp[s] ^ 0x80000000u);
}

__device__ inline uint32_t hash_pos(int t, int shift) {
  return ((uint32_t)t * 2654435761u) >> shift;  // Knuth multiplicative hash
}

__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(ResolveParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int k = p.k, S = p.S;
  int32_t* outb = p.out + (int64_t)b * k;
  const int32_t* tk = p.topk + (int64_t)b * k;
  const int r = p.req_idx[b];

  if (r < 0 || r >= p.R) {  // padding row
    for (int i = tid; i < k; i += kResolveThreads) outb[i] = -1;
    if (tid == 0) {
      p.plan_cnt[b] = 0;
      if (r >= p.R && p.stats) atomicAdd(&p.stats[4], 1ull);
    }
    return;
  }

  const int nraw = p.seq_lens[b];
  const int64_t n = (int64_t)nraw < p.max_seq_len ? (int64_t)nraw : p.max_seq_len;
  const int32_t c = (int32_t)((uint32_t)p.clk[r] + 1u);
  int32_t* st = p.st + (int64_t)r * S;
  int32_t* lru = p.lru + (int64_t)r * S;
  const int rowbase = r * S;
  const ResolveLds L = resolve_lds_layout(S, k);
  int* s_scr = (int*)(smem + L.off_scratch);

  if (nraw <= S) {  // fast path: slot == position, nothing copied
    int cnt = 0;
    for (int i = tid; i < k; i += kResolveThreads) {
      const int t = tk[i];
      if (t >= 0 && (int64_t)t < n) {
        outb[i] = rowbase + t;
        st[t] = t;
        lru[t] = c;
        ++cnt;
      } else {
        outb[i] = -1;
      }
    }
    int tot;
    block_exscan(cnt, s_scr, &tot);
    if (tid == 0) {
      p.clk[r] = c;
      p.plan_cnt[b] = 0;
      if (p.stats && tot) atomicAdd(&p.stats[3], (unsigned long long)tot);
    }
    return;
  }

  int32_t* s_tok = (int32_t*)(smem + L.off_tok);
  int32_t* s_stamp = (int32_t*)(smem + L.off_stamp);
  uint8_t* s_flag = (uint8_t*)(smem + L.off_flag);  // 0 candidate, 1 hit, 2 victim
  int32_t* e_tok = (int32_t*)(smem + L.off_etok);   // pending position or -1
  int32_t* m_entry = (int32_t*)(smem + L.off_mentry);
  int32_t* victim = (int32_t*)(smem + L.off_victim);
  int32_t* h_key = (int32_t*)(smem + L.off_hkey);
  int32_t* h_val = (int32_t*)(smem + L.off_hval);
  int32_t* e_hit = (int32_t*)(smem + L.off_ehit);
  uint64_t* s_sort = (uint64_t*)(smem + L.off_sort);
  const int H = L.hash_size;
  const int hshift = 32 - ilog2(H);

  for (int i = tid; i < H; i += kResolveThreads) {
    h_key[i] = -1;
    h_val[i] = INT_MAX;
  }
  for (int i = tid; i < k; i += kResolveThreads) e_hit[i] = INT_MAX;
  for (int s = tid; s < S; s += kResolveThreads) {  // stage the slot state
    s_tok[s] = st[s];
    s_stamp[s] = lru[s];
    s_flag[s] = 0;
  }
  __syncthreads();

  // Step 1: validity, resident pages, hash of the positions still pending.
  int n_res = 0, n_trip = 0;
  for (int i = tid; i < k; i += kResolveThreads) {
    const int t = tk[i];
    int pend = -1;
    if (t >= 0 && (int64_t)t < n) {
      bool resident = false;
      if (p.bt != nullptr) {
        const int pg = p.bt[(int64_t)r * p.max_pages + t / p.P];
        if (pg >= 0 && (int64_t)pg < p.resident_pages) {
          outb[i] = (int)((int64_t)p.R * S + (int64_t)pg * p.P + t % p.P);
          resident = true;
          ++n_res;
        } else if (pg >= 0) {
          ++n_trip;
        }
      }
      if (!resident) {
        pend = t;
        uint32_t h = hash_pos(t, hshift);
        while (true) {
          const int prev = atomicCAS(&h_key[h], -1, t);
          if (prev == -1 || prev == t) {
            atomicMin(&h_val[h], i);
            break;
          }
          h = (h + 1) & (H - 1);
        }
      }
    } else {
      outb[i] = -1;
    }
    e_tok[i] = pend;
  }
  __syncthreads();

  // Step 2: each slot holding a pending position marks that entry's hit slot
  // (the lowest such slot if the map were ever corrupted into duplicates).
  const int seg = (S + kResolveThreads - 1) / kResolveThreads;
  const int s0 = min(S, tid * seg), s1 = min(S, s0 + seg);
  for (int s = tid; s < S; s += kResolveThreads) {
    const int tok = s_tok[s];
    if (tok >= 0 && (int64_t)tok < n) {
      uint32_t h = hash_pos(tok, hshift);
      while (true) {
        const int key = h_key[h];
        if (key == tok) {
          atomicMin(&e_hit[h_val[h]], s);
          break;
        }
        if (key == -1) break;
        h = (h + 1) & (H - 1);
      }
    }
  }
  __syncthreads();

  // Step 3: hits (row ID, stamp refresh) and the misses in ascending index.
  const int segk = (k + kResolveThreads - 1) / kResolveThreads;
  const int i0 = min(k, tid * segk), i1 = min(k, i0 + segk);
  int n_hit = 0, my_miss = 0;
  for (int i = i0; i < i1; ++i) {
    if (e_tok[i] < 0) continue;
    const int s = e_hit[i];
    if (s != INT_MAX) {
      outb[i] = rowbase + s;
      lru[s] = c;
      s_flag[s] = 1;
      ++n_hit;
    } else {
      ++my_miss;
    }
  }
  int m_total;
  int mpos = block_exscan(my_miss, s_scr, &m_total);
  for (int i = i0; i < i1; ++i)
    if (e_tok[i] >= 0 && e_hit[i] == INT_MAX) m_entry[mpos++] = i;

  // Step 4: victims = the m_total smallest (occupied, stamp, slot) among
  // non-hit slots, in that order.  Each round takes the smallest remaining
  // (occupied, stamp) value and ranks its slots in slot order.
  int need = m_total, vbase = 0;
  for (int round = 0; round < kVictimRounds && need > 0; ++round) {
    uint64_t my = ~0ull;
    for (int s = s0; s < s1; ++s)
      if (s_flag[s] == 0) {
        const uint64_t kk = key33(s_tok, s_stamp, s);
        my = kk < my ? kk : my;
      }
    const uint64_t kmin = block_min_u64(my, (uint64_t*)s_scr);
    int cnt = 0;
    for (int s = s0; s < s1; ++s) cnt += (s_flag[s] == 0 && key33(s_tok, s_stamp, s) == kmin);
    int tot;
    int pos = block_exscan(cnt, s_scr, &tot);
    for (int s = s0; s < s1 && pos < need; ++s) {
      if (s_flag[s] == 0 && key33(s_tok, s_stamp, s) == kmin) {
        victim[vbase + pos] = s;
        s_flag[s] = 2;
        ++pos;
      }
    }
    const int take = tot < need ? tot : need;
    vbase += take;
    need -= take;
  }
  if (need > 0) {  // many distinct stamps among the victims: full sort
    __syncthreads();
    const int N = L.sort_size;
    for (int x = tid; x < N; x += kResolveThreads) {
      uint64_t v = ~0ull;
      if (x < S && s_flag[x] == 0) v = (key33(s_tok, s_stamp, x) << 16) | (uint64_t)x;
      s_sort[x] = v;
    }
    __syncthreads();
    for (int size = 2; size <= N; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int x = tid; x < N / 2; x += kResolveThreads) {
          const int lo = 2 * x - (x & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint64_t a = s_sort[lo], bb = s_sort[hi];
          if ((a > bb) == up) {
            s_sort[lo] = bb;
            s_sort[hi] = a;
          }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < need; j += kResolveThreads)
      victim[vbase + j] = (int)(s_sort[j] & 0xFFFFull);
  }
  __syncthreads();

  // Step 5: assign the j-th miss to the j-th victim and emit the plan.
  int64_t* psrc = p.plan_src + (int64_t)b * p.plan_stride;
  int32_t* pdst = p.plan_dst + (int64_t)b * p.plan_stride;
  const int64_t* locr = p.locs + (int64_t)r * p.max_seq_len;
  for (int j = tid; j < m_total; j += kResolveThreads) {
    const int i = m_entry[j];
    const int s = victim[j];
    const int t = e_tok[i];
    st[s] = t;
    lru[s] = c;
    const int row = rowbase + s;
    outb[i] = row;
    psrc[j] = locr[t];
    pdst[j] = row;
  }

  // Counters: one atomic per counter per workgroup.
  const int w = tid / kWave, ln = tid & (kWave - 1);
  const int a0 = wave_sum(n_hit), a1 = wave_sum(n_res), a2 = wave_sum(n_trip);
  if (ln == 0) {
    s_scr[w] = a0;
    s_scr[kResolveWaves + w] = a1;
    s_scr[2 * kResolveWaves + w] = a2;
  }
  __syncthreads();
  if (tid == 0) {
    int h = 0, rs = 0, tr = 0;
    for (int i = 0; i < kResolveWaves; ++i) {
      h += s_scr[i];
      rs += s_scr[kResolveWaves + i];
      tr += s_scr[2 * kResolveWaves + i];
    }
    p.plan_cnt[b] = m_total;
    p.clk[r] = c;
    if (p.stats) {
      if (h) atomicAdd(&p.stats[0], (unsigned long long)h);
      if (m_total) atomicAdd(&p.stats[1], (unsigned long long)m_total);
      if (rs) atomicAdd(&p.stats[2], (unsigned long long)rs);
      if (tr) atomicAdd(&p.stats[4], (unsigned long long)tr);
    }
  }
}

}  // namespace

hipError_t launch_resolve(const ResolveParams& p, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  const ResolveLds L = resolve_lds_layout(p.S, p.k);
  hipLaunchKernelGGL(resolve_kernel, dim3(batch), dim3(kResolveThreads), L.total, stream, p);
  return hipGetLastError();
}

hipError_t prepare_resolve(size_t lds_bytes) {
  return hipFuncSetAttribute((const void*)resolve_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_bytes);
}

}  // namespace hisparse
