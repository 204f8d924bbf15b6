// resolve.hip -- the resolver's plan kernel for gfx950.
//
// One workgroup of 1024 threads (16 wavefronts) per batch row.  Thread t owns
// a contiguous run of SPT slots and a contiguous run of KPT top-k entries, so
// "ascending slot" and "ascending top-k index" are thread order and every
// rank below is a block-wide exclusive scan.  Slot tokens and stamps stay in
// registers; LDS holds an open-addressing table of the pending positions
// (one 64-bit word per cell: position << 32 | top-k index), the per-entry hit
// slot, the miss and victim lists, and per-wave partials.  Steps:
//   1. validity and the resident short-circuit; pending positions are
//      inserted into the table;
//   2. each slot holding a pending position marks that entry's hit slot (the
//      lowest slot if the map was corrupted into duplicates);
//   3. hits get their row ID and a refreshed stamp; misses are listed in
//      ascending top-k index with their host rows (loaded as soon as each
//      miss is known); a slot learns it is a hit slot from its entry;
//   4. victims: rounds of block-wide minimum over the candidates' (occupied,
//      stamp) keys, each round taking the slots of the minimum key in slot
//      order; if a few rounds do not cover every miss, a bitonic LDS sort of
//      the remaining candidates finishes the ranking;
//   5. the j-th miss takes the j-th victim: token, stamp, row ID and one
//      (host row, device row) entry of the compact miss plan;
//   6. (COPY instances) the workgroup copies its own misses from the pinned
//      host pools into every layer, one wavefront per row, so each request's
//      copy starts as soon as its plan exists and no second launch is needed;
//      each wavefront's first rows are loaded before step 4, so the host link
//      is busy while the victims are ranked.
// Resolution order and phases: "vLLM HiSparse 本地 KV 卸载架构" (hot-row lookup
// and LRU) and "vLLM Hybrid HiSparse 源码实现分析" section 7.2; fast path
// (seq_len <= S: slot == position, nothing moves): the per-step flow of the
// gogongxt.com HiSparse page.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

constexpr uint64_t kEmptyCell = ~0ull;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu4;  // 16 bytes of global memory
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// N consecutive int32 from `base` as 16-byte (or N*4-byte) vector loads; the
// caller guarantees the alignment.
template <int N>
__device__ inline void load_run(const int32_t* base, int (&v)[N]) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const i32x4 x = ((const i32x4*)base)[q];
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const i32x2 x = *(const i32x2*)base;
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = base[0];
  }
}

// N consecutive int32 to `base` as 16-byte (or N*4-byte) vector stores.
template <int N>
__device__ inline void store_run(int32_t* base, const int (&v)[N]) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      ((i32x4*)base)[q] = i32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
  } else if constexpr (N == 2) {
    *(i32x2*)base = i32x2{v[0], v[1]};
  } else {
    base[0] = v[0];
  }
}

__device__ inline int lane_prefix(uint64_t m) {  // popcount of m below this lane
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// One DPP step of a wavefront minimum: lanes whose source is outside the
// pattern (or whose row is masked off) see the identity ~0.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_min_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFF, (int)v, CTRL, ROWS, 0xF, false);
  return o < v ? o : v;
}

// Minimum of a 32-bit value over the 64 lanes, wave-uniform: prefix minima
// within each row of 16 (row_shr 1, 2, 4, 8), then row 0 into row 1 and
// row 2 into row 3 (row_bcast:15), then rows 0-1 into rows 2-3
// (row_bcast:31); lane 63 holds the result.
__device__ inline uint32_t wave_min_u32(uint32_t v) {
  v = dpp_min_step<0x111, 0xF>(v);
  v = dpp_min_step<0x112, 0xF>(v);
  v = dpp_min_step<0x114, 0xF>(v);
  v = dpp_min_step<0x118, 0xF>(v);
  v = dpp_min_step<0x142, 0xA>(v);
  v = dpp_min_step<0x143, 0xC>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Minimum of victim keys (occupied << 32 | biased stamp, or ~0) over the
// wavefront: the occupied bit by ballot, then the stamps of the lanes at
// that bit by a 32-bit minimum.
__device__ inline uint64_t wave_min_key(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32);  // 0 empty, 1 occupied, ~0 none
  const bool any_empty = __ballot(hi == 0) != 0;
  const bool any_occ = __ballot(hi == 1) != 0;
  if (!any_empty && !any_occ) return ~0ull;
  const uint32_t want = any_empty ? 0u : 1u;
  const uint32_t m = wave_min_u32(hi == want ? (uint32_t)v : 0xFFFFFFFFu);
  return ((uint64_t)want << 32) | m;
}

// One DPP step of an inclusive wavefront prefix sum: lanes whose source is
// outside the pattern (or whose row is masked off) add 0.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_add_step(uint32_t v) {
  return v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes: within each row of 16 (row_shr 1,
// 2, 4, 8), then the last lane of row 0 into row 1 and of row 2 into row 3
// (row_bcast:15), then lane 31 into rows 2-3 (row_bcast:31).
__device__ inline uint32_t wave_inclusive_sum(uint32_t v) {
  v = dpp_add_step<0x111, 0xF>(v);
  v = dpp_add_step<0x112, 0xF>(v);
  v = dpp_add_step<0x114, 0xF>(v);
  v = dpp_add_step<0x118, 0xF>(v);
  v = dpp_add_step<0x142, 0xA>(v);
  v = dpp_add_step<0x143, 0xC>(v);
  return v;
}

// Sum over the wavefront of small per-lane counts (< 2^BITS), by ballots.
template <int BITS>
__device__ inline int wave_sum_small(int v) {
  int sum = 0;
#pragma unroll
  for (int q = 0; q < BITS; ++q) sum += __popcll(__ballot((v >> q) & 1)) << q;
  return sum;
}

// Block-wide exclusive prefix sum of small per-thread counts (< 2^BITS) in
// thread order, with one barrier.  `buf` holds 16 ints used by this call
// site only.
template <int BITS>
__device__ inline int block_exscan_small(int c, int* buf, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  int pre = 0, wt = 0;
#pragma unroll
  for (int q = 0; q < BITS; ++q) {
    const uint64_t m = __ballot((c >> q) & 1);
    pre += lane_prefix(m) << q;
    wt += __popcll(m) << q;
  }
  if (lane == 0) buf[wid] = wt;
  lds_barrier();
  // Lane w holds wave w's total; one prefix sum gives every wave its base
  // (one LDS read per lane instead of kResolveWaves dependent reads).
  const uint32_t inc = wave_inclusive_sum(lane < kResolveWaves ? (uint32_t)buf[lane] : 0u);
  *total = __builtin_amdgcn_readlane((int)inc, 63);
  const int base = wid > 0 ? __builtin_amdgcn_readlane((int)inc, wid - 1) : 0;
  return base + pre;
}

// Block-wide minimum of victim keys with one barrier; `buf` holds 16 u64 for
// this call site.
__device__ inline uint64_t block_min_key(uint64_t v, uint64_t* buf) {
  const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
  const uint64_t wm = wave_min_key(v);
  if (lane == 0) buf[wid] = wm;
  lds_barrier();
  return wave_min_key(lane < kResolveWaves ? buf[lane] : ~0ull);  // lane w: wave w's minimum
}

__device__ inline uint32_t hash_pos(int t, int shift) {
  return ((uint32_t)t * 2654435761u) >> shift;  // Knuth multiplicative hash
}

constexpr int bits_for(int v) { return v <= 1 ? 1 : 1 + bits_for(v >> 1); }

// Scratch buffers (16 entries each) of the call sites, in ints.
enum : int {
  kScrFast = 0,
  kScrMiss = 16,
  kScrStats = 32,        // 3 x 16
  kScrRoundScan = 80,    // kVictimRounds x 16
  kScrRoundMin = 160,    // kVictimRounds x 16 u64 (= 32 ints each), 8-byte aligned
  kScrInts = 160 + 32 * kVictimRounds
};
static_assert(kScrInts == kResolveScratchInts, "scratch layout");

// COPY: the workgroup also copies its misses into p.copy_layers layers.
// VEC: each thread's slot-state run is loaded as vectors.
template <int SPT, int KPT, bool COPY, bool VEC>
__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(ResolveParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  const int k = p.k, S = p.S;
  int32_t* outb = p.out + (int64_t)b * k;
  const int32_t* tk = p.topk + (int64_t)b * k;
  const int r = p.req_idx[b];
  const int nraw = p.seq_lens[b];

  // This thread's top-k entries, loaded before anything depends on r.  The
  // loads use clamped (always in-range) indices so that they issue back to
  // back without per-load branches; entries past k hold a copy of entry k-1
  // and are skipped wherever used.
  const int i0 = tid * KPT;
  int tr[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) tr[j] = -1;
  if (k > 0) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) tr[j] = tk[min(i0 + j, k - 1)];
  }

  if (r < 0 || r >= p.R) {  // padding row
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (i0 + j < k) outb[i0 + j] = -1;
    if (tid == 0) {
      p.plan_cnt[b] = 0;
      if (r >= p.R && p.stats) atomicAdd(&p.stats[4], 1ull);
    }
    return;
  }

  const int64_t n = (int64_t)nraw < p.max_seq_len ? (int64_t)nraw : p.max_seq_len;
  const int32_t c = (int32_t)((uint32_t)p.clk[r] + 1u);
  int32_t* st = p.st + (int64_t)r * S;
  int32_t* lru = p.lru + (int64_t)r * S;
  const int rowbase = r * S;
  const ResolveLds& L = p.lds;
  int* scr = (int*)(smem + L.off_scratch);

  if (nraw <= S) {  // fast path: slot == position, nothing copied
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = i0 + j;
      if (i >= k) continue;
      const int t = tr[j];
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
    block_exscan_small<bits_for(KPT)>(cnt, scr + kScrFast, &tot);
    if (tid == 0) {
      p.clk[r] = c;
      p.plan_cnt[b] = 0;
      if (p.stats && tot) atomicAdd(&p.stats[3], (unsigned long long)tot);
    }
    return;
  }

  // Slot state of this thread's slots (registers); slots past S hold a copy
  // of slot S-1 and are excluded wherever used.
  const int s0 = tid * SPT;
  int sr[SPT], lr[SPT];
  // VEC (S % SPT == 0, aligned rows): two vector runs.  A separate instance,
  // not a branch: merging the two load paths would make the compiler wait
  // for the loads at the merge.
  if constexpr (VEC) {
    const int sv = min(s0, S - SPT);
    load_run<SPT>(st + sv, sr);
    load_run<SPT>(lru + sv, lr);
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int s = min(s0 + j, S - 1);
      sr[j] = st[s];
      lr[j] = lru[s];
    }
  }

  // Block-table entries of this thread's positions, at in-range indices,
  // issued with the slot-state loads so that both round trips overlap.
  int pgs[KPT];
  if (p.bt != nullptr) {
    const int32_t* btr = p.bt + (int64_t)r * p.max_pages;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int t = tr[j];
      const bool v = t >= 0 && (int64_t)t < n;
      pgs[j] = btr[v ? t / p.P : 0];
    }
  }

  uint64_t* H = (uint64_t*)(smem + L.off_hash);
  int32_t* e_hit = (int32_t*)(smem + L.off_ehit);
  int32_t* e_tok = (int32_t*)(smem + L.off_etok);
  int32_t* m_entry = (int32_t*)(smem + L.off_mentry);
  int32_t* victim = (int32_t*)(smem + L.off_victim);
  // Host row of the j-th miss.  Host pools hold fewer than 2^31 rows (checked
  // at init), so a row outside [0, 2^31) is kept as -1: out of range either way.
  int32_t* m_h = (int32_t*)(smem + L.off_mhost);
  uint64_t* s_sort = (uint64_t*)(smem + L.off_sort);
  const int HS = L.hash_size;
  const int hshift = 32 - ilog2(HS);

  for (int x = tid; x < HS; x += kResolveThreads) H[x] = kEmptyCell;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (i0 + j < k) e_hit[i0 + j] = INT_MAX;
  // Barriers below order LDS only: no thread reads global memory that another
  // thread of the workgroup wrote, so the slot-state loads stay in flight
  // through step 1 and the row-ID and stamp stores never hold a barrier.
  lds_barrier();

  // Step 1: validity, resident pages, table of pending positions.
  int n_res = 0, n_trip = 0;
  unsigned pend = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = i0 + j;
    if (i >= k) continue;
    const int t = tr[j];
    if (t < 0 || (int64_t)t >= n) {
      outb[i] = -1;
      continue;
    }
    if (p.bt != nullptr) {
      const int pg = pgs[j];
      if (pg >= 0 && (int64_t)pg < p.resident_pages) {
        outb[i] = (int)((int64_t)p.R * S + (int64_t)pg * p.P + t % p.P);
        ++n_res;
        continue;
      }
      if (pg >= 0) ++n_trip;
    }
    pend |= 1u << j;
    e_tok[i] = t;
    const uint64_t cell = ((uint64_t)(uint32_t)t << 32) | (uint32_t)i;
    uint32_t h = hash_pos(t, hshift);
    while (true) {
      const uint64_t prev = atomicCAS((unsigned long long*)&H[h], kEmptyCell, cell);
      if (prev == kEmptyCell || (int)(prev >> 32) == t) break;  // inserted, or a repeat
      h = (h + 1) & (HS - 1);
    }
  }
  lds_barrier();

  // Step 2: probe the table with every slot's token; the SPT probes of a
  // thread advance together so a wavefront waits for its longest chain once.
  int hidx[SPT];  // top-k index of the pending entry this slot's token matches, or -1
  {
    uint32_t hh[SPT];
    uint64_t hv[SPT];
    unsigned live = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int tok = sr[j];
      const bool ok = (s0 + j < S) && tok >= 0 && (int64_t)tok < n;
      hh[j] = hash_pos(tok, hshift);
      hv[j] = ok ? H[hh[j]] : kEmptyCell;
      if (ok) live |= 1u << j;
    }
    while (true) {
      unsigned next = 0;
#pragma unroll
      for (int j = 0; j < SPT; ++j)
        if ((live & (1u << j)) && hv[j] != kEmptyCell && (int)(hv[j] >> 32) != sr[j])
          next |= 1u << j;
      if (next == 0) break;
#pragma unroll
      for (int j = 0; j < SPT; ++j)
        if (next & (1u << j)) {
          hh[j] = (hh[j] + 1) & (HS - 1);
          hv[j] = H[hh[j]];
        }
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      hidx[j] = ((live & (1u << j)) && hv[j] != kEmptyCell) ? (int)(uint32_t)hv[j] : -1;
      if (hidx[j] >= 0) atomicMin(&e_hit[hidx[j]], s0 + j);
    }
  }
  lds_barrier();

  // Step 3: hits and the ordered miss list.  A miss's host row is loaded as
  // soon as the miss is known; it travels with the list.
  const int64_t* locr = p.locs + (int64_t)r * p.max_seq_len;
  int n_hit = 0, my_miss = 0;
  unsigned missbits = 0;
  int32_t hm[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    hm[j] = -1;
    if (!(pend & (1u << j))) continue;
    const int i = i0 + j;
    const int s = e_hit[i];
    if (s != INT_MAX) {
      outb[i] = rowbase + s;  // the slot's owner refreshes its stamp
      ++n_hit;
    } else {
      missbits |= 1u << j;
      ++my_miss;
      const int64_t h = locr[tr[j]];
      hm[j] = (h >= 0 && h <= INT_MAX) ? (int32_t)h : -1;
    }
  }
  {
    const int a0 = wave_sum_small<bits_for(KPT)>(n_hit);
    const int a1 = wave_sum_small<bits_for(KPT)>(n_res);
    const int a2 = wave_sum_small<bits_for(KPT)>(n_trip);
    if (lane == 0) {
      scr[kScrStats + wid] = a0;
      scr[kScrStats + 16 + wid] = a1;
      scr[kScrStats + 32 + wid] = a2;
    }
  }
  int m_total;
  int mpos = block_exscan_small<bits_for(KPT)>(my_miss, scr + kScrMiss, &m_total);
  // Slots: the hit slot of an entry is the one that entry's e_hit names.
  unsigned hitm = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if (hidx[j] >= 0 && e_hit[hidx[j]] == s0 + j) hitm |= 1u << j;

  // The miss list; the fused instance also needs the host rows now (for the
  // rows loaded ahead), the plan-only instance writes them after the victims
  // are ranked, so the loads never hold a barrier.
  const int mpos0 = mpos;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (missbits & (1u << j)) {
      if (COPY) m_h[mpos] = hm[j];
      m_entry[mpos++] = i0 + j;
    }

  // Fused copy, first rows: each wavefront loads its first kCopyRowsInFlight
  // rows of the first layer now, so the host link already works while the
  // victims are ranked; they are stored once their slots are known.
  constexpr int RIF = kCopyRowsInFlight;
  u32x4 pre[RIF];
  const bool have_pre = COPY && m_total > 0 && p.units <= kWave;
  if (have_pre) {
    lds_barrier();  // the miss list of every wavefront
#pragma unroll
    for (int q = 0; q < RIF; ++q) {
      pre[q] = u32x4{0u, 0u, 0u, 0u};
      const int j = wid + q * kResolveWaves;
      if (j < m_total) {
        const int64_t h = __builtin_amdgcn_readfirstlane(m_h[j]);
        const bool ok = h >= 0 && h < p.host_rows[0];
        const gu4* src = ok ? (const gu4*)p.host_pool[0] + h * p.units : (const gu4*)p.zero_row;
        if (lane < p.units) pre[q] = src[lane];
      }
    }
  }

  // Step 4: victims, in (occupied, stamp, slot) order among non-hit slots.
  uint64_t key[SPT];
  unsigned cand = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    key[j] = ((uint64_t)(sr[j] >= 0 ? 1u : 0u) << 32) | (uint64_t)((uint32_t)lr[j] ^ 0x80000000u);
    if (s0 + j < S && !(hitm & (1u << j))) cand |= 1u << j;
  }
  int vr[SPT];  // rank of this slot among the victims, or -1
#pragma unroll
  for (int j = 0; j < SPT; ++j) vr[j] = -1;
  int need = m_total, vbase = 0;
#pragma unroll 1
  for (int round = 0; round < kVictimRounds && need > 0; ++round) {
    uint64_t my = ~0ull;
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if ((cand & (1u << j)) && key[j] < my) my = key[j];
    const uint64_t kmin =
        block_min_key(my, (uint64_t*)(scr + kScrRoundMin + 32 * round));
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) cnt += ((cand & (1u << j)) && key[j] == kmin) ? 1 : 0;
    int tot;
    int pos = block_exscan_small<bits_for(SPT)>(cnt, scr + kScrRoundScan + 16 * round, &tot);
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      if ((cand & (1u << j)) && key[j] == kmin) {
        if (pos < need) {
          vr[j] = vbase + pos;
          cand &= ~(1u << j);
        }
        ++pos;
      }
    }
    const int take = tot < need ? tot : need;
    vbase += take;
    need -= take;
  }
  if (need > 0) {  // many distinct stamps among the victims: sort the rest
    const int N = L.sort_size;
    lds_barrier();  // the table region is reused for the sort
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int s = s0 + j;
      if (s < N) s_sort[s] = (cand & (1u << j)) ? ((key[j] << 16) | (uint64_t)s) : ~0ull;
    }
    for (int x = tid + kResolveThreads * SPT; x < N; x += kResolveThreads) s_sort[x] = ~0ull;
    lds_barrier();
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
        lds_barrier();
      }
    }
    for (int j = tid; j < need; j += kResolveThreads) {
      const int s = (int)(s_sort[j] & 0xFFFFull);
      victim[vbase + j] = s < S ? s : S - 1;  // always < S: candidates >= misses
    }
    // The sorted victims' ranks by slot, in the (now dead) sort region.
    int32_t* vrank = (int32_t*)s_sort;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (s0 + j < S) vrank[s0 + j] = -1;
    lds_barrier();
    for (int j = tid; j < need; j += kResolveThreads) vrank[victim[vbase + j]] = vbase + j;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (cand & (1u << j)) {
        const int v = vrank[s0 + j];
        if (v >= 0) vr[j] = v;
      }
  }
  if (!COPY) {
    int mp = mpos0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (missbits & (1u << j)) m_h[mp++] = hm[j];
  }
  lds_barrier();

  // Step 5: the victim of rank j takes the j-th miss: its owner sets token
  // and row ID and writes one entry of the compact plan.  The fused copy keeps
  // its own copy of the plan in the (now dead) table region.  Then every
  // thread writes its slot run back once: stamps of hit and victim slots,
  // tokens of victim slots (vector stores, not one scattered store per slot).
  int64_t* psrc = p.plan_src + (int64_t)b * p.plan_stride;
  int32_t* pdst = p.plan_dst + (int64_t)b * p.plan_stride;
  int64_t* f_src = (int64_t*)(smem + L.off_hash);          // [k]
  int32_t* f_dst = (int32_t*)(smem + L.off_hash + 8 * (size_t)k);  // [k]
  unsigned vict = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    if (vr[j] < 0) continue;
    vict |= 1u << j;
    const int v = vr[j];
    const int i = m_entry[v];
    sr[j] = e_tok[i];
    const int row = rowbase + s0 + j;
    outb[i] = row;
    const int64_t h = m_h[v];  // -1 for a row outside [0, 2^31)
    psrc[v] = h;
    pdst[v] = row;
    if (COPY) {
      f_src[v] = h;
      f_dst[v] = row;
    }
  }
  const unsigned touched = hitm | vict;
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if (touched & (1u << j)) lr[j] = c;
  if constexpr (VEC) {
    if (s0 < S) {
      if (touched) store_run<SPT>(lru + s0, lr);
      if (vict) store_run<SPT>(st + s0, sr);
    }
  } else {
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      if (touched & (1u << j)) lru[s0 + j] = c;
      if (vict & (1u << j)) st[s0 + j] = sr[j];
    }
  }

  // Fused miss copy: one wavefront per (layer, miss) row, lane l carrying
  // 16-byte unit l, kCopyRowsInFlight rows in flight per wavefront.  Row
  // indices are wave-uniform (scalar), and the per-layer pointers come from
  // the kernel arguments.  A host row out of range reads the zero row instead
  // and counts one tripwire, as the separate copy kernel does.  Past the end
  // of the list a wavefront repeats its first row of the batch (the same
  // bytes again), so every load is unconditional.
  int copy_trips = 0;
  if (COPY && m_total > 0) {
    lds_barrier();
    const int U = p.units;
    const int total = m_total * p.copy_layers;
    const int wu = __builtin_amdgcn_readfirstlane(wid);
#pragma unroll 1
    for (int u = wu; u < total; u += RIF * kResolveWaves) {
      const bool first = u == wu;
      const gu4* src[RIF];
      gu4* dst[RIF];
#pragma unroll
      for (int q = 0; q < RIF; ++q) {
        const bool real = u + q * kResolveWaves < total;
        const int uq = real ? u + q * kResolveWaves : u;
        const int l = uq / m_total, j = uq - l * m_total;
        const int64_t h = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)f_src[j]) |
                          ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(f_src[j] >> 32)) << 32);
        const int d = __builtin_amdgcn_readfirstlane(f_dst[j]);
        const bool ok = h >= 0 && h < p.host_rows[l];
        src[q] = ok ? (const gu4*)p.host_pool[l] + h * U : (const gu4*)p.zero_row;
        dst[q] = (gu4*)p.dev_pool[l] + (int64_t)d * U;
        copy_trips += (real && !ok) ? 1 : 0;
      }
      for (int part = lane; part < U; part += kWave) {
        u32x4 v[RIF];
#pragma unroll
        for (int q = 0; q < RIF; ++q) {
          // rows of the first layer that were loaded ahead (one unit per lane)
          if (have_pre && first && u + q * kResolveWaves < m_total) v[q] = pre[q];
          else v[q] = src[q][part];
        }
#pragma unroll
        for (int q = 0; q < RIF; ++q) dst[q][part] = v[q];
      }
    }
  }

  if (wid == 0) {  // lane w of wave 0 adds wave w's counters
    const bool in = lane < kResolveWaves;
    const int h = __builtin_amdgcn_readlane(
        (int)wave_inclusive_sum(in ? (uint32_t)scr[kScrStats + lane] : 0u), 63);
    const int rs = __builtin_amdgcn_readlane(
        (int)wave_inclusive_sum(in ? (uint32_t)scr[kScrStats + 16 + lane] : 0u), 63);
    const int tr2 = __builtin_amdgcn_readlane(
        (int)wave_inclusive_sum(in ? (uint32_t)scr[kScrStats + 32 + lane] : 0u), 63);
    if (lane == 0) {
      p.plan_cnt[b] = m_total;
      p.clk[r] = c;
      if (p.stats) {
        if (h) atomicAdd(&p.stats[0], (unsigned long long)h);
        if (m_total) atomicAdd(&p.stats[1], (unsigned long long)m_total);
        if (rs) atomicAdd(&p.stats[2], (unsigned long long)rs);
        if (tr2) atomicAdd(&p.stats[4], (unsigned long long)tr2);
      }
    }
  }
  if (copy_trips && lane == 0 && p.stats) atomicAdd(&p.stats[4], (unsigned long long)copy_trips);
}

template <int SPT, int KPT>
hipError_t launch_t(const ResolveParams& p, int batch, size_t lds, hipStream_t stream) {
  const dim3 g(batch), t(kResolveThreads);
  if (p.copy_layers > 0) {
    if (p.vec_state) hipLaunchKernelGGL((resolve_kernel<SPT, KPT, true, true>), g, t, lds, stream, p);
    else hipLaunchKernelGGL((resolve_kernel<SPT, KPT, true, false>), g, t, lds, stream, p);
  } else {
    if (p.vec_state) hipLaunchKernelGGL((resolve_kernel<SPT, KPT, false, true>), g, t, lds, stream, p);
    else hipLaunchKernelGGL((resolve_kernel<SPT, KPT, false, false>), g, t, lds, stream, p);
  }
  return hipGetLastError();
}

template <int SPT>
hipError_t launch_k(const ResolveParams& p, int batch, size_t lds, hipStream_t stream, int kpt) {
  switch (kpt) {
    case 1: return launch_t<SPT, 1>(p, batch, lds, stream);
    case 2: return launch_t<SPT, 2>(p, batch, lds, stream);
    case 4: return launch_t<SPT, 4>(p, batch, lds, stream);
    default: return launch_t<SPT, 8>(p, batch, lds, stream);
  }
}

template <int SPT, int KPT>
hipError_t set_attr() {
  const void* fns[4] = {(const void*)resolve_kernel<SPT, KPT, false, false>,
                        (const void*)resolve_kernel<SPT, KPT, false, true>,
                        (const void*)resolve_kernel<SPT, KPT, true, false>,
                        (const void*)resolve_kernel<SPT, KPT, true, true>};
  for (const void* f : fns) {
    const hipError_t e =
        hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBudget);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int SPT>
hipError_t set_attr_k() {
  hipError_t e = set_attr<SPT, 1>();
  if (e == hipSuccess) e = set_attr<SPT, 2>();
  if (e == hipSuccess) e = set_attr<SPT, 4>();
  if (e == hipSuccess) e = set_attr<SPT, 8>();
  return e;
}

}  // namespace

hipError_t launch_resolve(ResolveParams p, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  p.lds = resolve_lds_layout(p.S, p.k);
  const size_t lds = p.lds.total;
  const int spt = resolve_slots_per_thread(p.S);
  const int kpt = resolve_entries_per_thread(p.k);
  auto aligned = [](const void* q, int per) {
    const uintptr_t a = (uintptr_t)4 * (uintptr_t)(per < 4 ? per : 4);
    return ((uintptr_t)q % a) == 0;
  };
  p.vec_state = (p.S % spt == 0 && aligned(p.st, spt) && aligned(p.lru, spt)) ? 1 : 0;
  switch (spt) {
    case 1: return launch_k<1>(p, batch, lds, stream, kpt);
    case 2: return launch_k<2>(p, batch, lds, stream, kpt);
    case 4: return launch_k<4>(p, batch, lds, stream, kpt);
    case 8: return launch_k<8>(p, batch, lds, stream, kpt);
    default: return launch_k<16>(p, batch, lds, stream, kpt);
  }
}

hipError_t prepare_resolve(size_t) {
  hipError_t e = set_attr_k<1>();
  if (e == hipSuccess) e = set_attr_k<2>();
  if (e == hipSuccess) e = set_attr_k<4>();
  if (e == hipSuccess) e = set_attr_k<8>();
  if (e == hipSuccess) e = set_attr_k<16>();
  return e;
}

}  // namespace hisparse
