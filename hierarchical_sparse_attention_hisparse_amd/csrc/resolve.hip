// resolve.hip -- the resolver's plan kernel for gfx950.
//
// One workgroup of 1024 threads (16 wavefronts) per batch row.  Thread t owns
// a contiguous run of SPT slots and a contiguous run of KPT top-k entries, so
// "ascending slot" and "ascending top-k index" are thread order.  Slot tokens
// and stamps stay in registers; LDS holds an open-addressing table of the
// pending positions (32-bit cells in buckets of 4, with each cell's top-k
// index in a parallel 16-bit array), the per-entry hit slot, the miss list,
// the victim ranking's bitmaps and per-wave partials.  Steps:
//   1. validity and the resident short-circuit; pending positions are
//      inserted into the table;
//   2. each slot holding a pending position marks that entry's hit slot (the
//      lowest slot if the map was corrupted into duplicates);
//   3. hits get their row ID and a refreshed stamp; misses load their host
//      rows; a slot learns it is a hit slot from its entry;
//   4. the misses are listed in ascending top-k index; victims are ranked in
//      (occupied, stamp, slot) order by windows of consecutive keys: one
//      slot bitmap per key, popcount prefixes over each bitmap's words, and
//      a candidate's exact rank from those (three barriers per window; keys
//      spread over more windows fall back to a bitonic sort);
//   5. the j-th miss takes the j-th victim: token, stamp, row ID and one
//      (host row, device row) entry of the compact miss plan;
//   6. (COPY instances) the workgroup copies its own misses from the pinned
//      host pools into every layer, one wavefront per row, so each request's
//      copy starts as soon as its plan exists and no second launch is needed;
//      each wavefront's first rows are loaded before the ranks are known, so
//      the host link is busy while the victims are ranked.
// Resolution order and phases: "vLLM HiSparse 本地 KV 卸载架构" (hot-row lookup
// and LRU) and "vLLM Hybrid HiSparse 源码实现分析" section 7.2; fast path
// (seq_len <= S: slot == position, nothing moves): the per-step flow of the
// gogongxt.com HiSparse page.
#include <limits.h>

#include "common.h"
#include "kernels.h"

namespace hisparse {

#ifdef HISPARSE_PHASE_TRACE
// Phase trace (diagnostic build only): lane 0 of each wavefront of the batch
// rows below kTraceRows stores the shader clock and the 100 MHz real-time
// counter at each phase point; point 8 holds the ranking windows used and
// whether the sort fallback ran.
__device__ unsigned long long g_phase_trace[kTraceRows][kResolveWaves][kTracePoints][2];
#define PHASE_POINT(q)                                                         \
  do {                                                                         \
    if (lane == 0 && b < kTraceRows) {                                         \
      g_phase_trace[b][wid][q][0] = (unsigned long long)clock64();             \
      g_phase_trace[b][wid][q][1] = (unsigned long long)wall_clock64();        \
    }                                                                          \
  } while (0)
#define PHASE_INFO(nwin, sorted)                                               \
  do {                                                                         \
    if (lane == 0 && b < kTraceRows) {                                         \
      g_phase_trace[b][wid][8][0] = (unsigned long long)(nwin);                \
      g_phase_trace[b][wid][8][1] = (unsigned long long)(sorted);              \
    }                                                                          \
  } while (0)
#else
#define PHASE_POINT(q) \
  do {                 \
  } while (0)
#define PHASE_INFO(nwin, sorted) \
  do {                           \
  } while (0)
#endif

namespace {

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

__device__ inline uint32_t hash_pos(int t, int shift) {
  return ((uint32_t)t * 2654435761u) >> shift;  // Knuth multiplicative hash
}

constexpr int bits_for(int v) { return v <= 1 ? 1 : 1 + bits_for(v >> 1); }

// A host row as int32 for the fused copy's LDS list: host pools hold fewer
// than 2^31 rows (checked at init), so a row outside [0, 2^31) becomes -1,
// out of range either way.
__device__ inline int32_t host_row32(int64_t h) { return (h >= 0 && h <= INT_MAX) ? (int32_t)h : -1; }

// Scratch buffers of the call sites, in ints: per-wave partials (16 each)
// and the window's candidate count per key.  kScrKey0 shares the fast path's
// ints: a row takes one path or the other.
enum : int {
  kScrFast = 0,
  kScrKey0 = 0,          // candidates at each wave's smallest key (step 3)
  kScrMiss = 16,
  kScrStats = 32,        // 3 x 16
  kScrMin = 80,          // 2 x 16 u64 (= 64 ints), 8-byte aligned: double-buffered per window
  kScrBtot = 144,        // kMaxRankBins
  kScrInts = 176
};
static_assert(kScrInts == kResolveScratchInts, "scratch layout");
static_assert(kScrBtot + kMaxRankBins <= kScrInts, "scratch layout");

// COPY: the workgroup also copies its misses into p.copy_layers layers.
// VEC: each thread's slot-state run is loaded as vectors.
// PAGED: a block table maps resident pages (p.bt not null).  A separate
// instance: the rows without one then carry no page code at all.
template <int SPT, int KPT, bool COPY, bool VEC, bool PAGED>
__global__ __launch_bounds__(kResolveThreads) void resolve_kernel(ResolveParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  PHASE_POINT(0);
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
  int32_t* st = p.st + (int64_t)r * S;
  int32_t* lru = p.lru + (int64_t)r * S;
  const int rowbase = r * S;
  const ResolveLds& L = p.lds;
  int* scr = (int*)(smem + L.off_scratch);

  if (nraw <= S) {  // fast path: slot == position, nothing copied
    const int32_t c = (int32_t)((uint32_t)p.clk[r] + 1u);
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

  // The request's clock, through a vector load (a zero the compiler cannot
  // see through makes its address a vector one): the barriers wait for every
  // scalar load in flight, so as a scalar load it would hold the first one
  // for a second dependent round trip.  It is first used at the end.
  int vzero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  const int32_t clk_now = p.clk[r + vzero];
  // The fill-count increment of step 1, in a register defined before the
  // block-table loads below: were it placed after them, it could share a
  // register with one of those loads, and the rows without a block table
  // would then wait for every load in flight (slot state included) before
  // their inserts.
  int vone;
  asm volatile("v_mov_b32 %0, 1" : "=v"(vone));

  // Block-table entries of this thread's positions, at in-range indices,
  // issued with the slot-state loads so that both round trips overlap.
  int pgs[KPT];
  if constexpr (PAGED) {
    const int32_t* btr = p.bt + (int64_t)r * p.max_pages;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int t = tr[j];
      const bool v = t >= 0 && (int64_t)t < n;
      // (a power-of-two page size divides by a shift: a uniform branch)
      pgs[j] = btr[v ? (p.P_shift >= 0 ? t >> p.P_shift : t / p.P) : 0];
    }
  }

  // Table of the pending positions: 32-bit cells (a position, -1 = empty)
  // in buckets of kBucketCells, with the top-k index of each cell in a
  // parallel 16-bit array.  A position hashes to a bucket and takes the cell
  // that the bucket's fill count names (one atomic add); past a full bucket
  // it tries the next.  So the taken cells of a bucket are a prefix of it,
  // and a position absent from a bucket whose last cell is free is absent
  // from the table.  Probes read whole buckets (16-byte reads) and read the
  // matched cell's index once, after their loop.
  int32_t* Hc = (int32_t*)(smem + L.off_hash);
  uint16_t* Hi = (uint16_t*)(smem + L.off_hidx);
  int32_t* Hn = (int32_t*)(smem + L.off_hcnt);
  int32_t* e_hit = (int32_t*)(smem + L.off_ehit);
  int32_t* e_tok = (int32_t*)(smem + L.off_etok);
  int32_t* m_entry = (int32_t*)(smem + L.off_mentry);
  int32_t* victim = (int32_t*)(smem + L.off_victim);
  // Host row of the j-th miss for the fused copy (see host_row32).
  int32_t* m_h = (int32_t*)(smem + L.off_mhost);
  uint64_t* s_sort = (uint64_t*)(smem + L.off_sort);
  const int HS = L.hash_size;
  const int NBK = HS / kBucketCells;        // buckets (a power of two >= 16)
  const int bshift = 32 - ilog2(NBK);

  for (int x = tid; x < HS / 4; x += kResolveThreads) ((i32x4*)Hc)[x] = i32x4{-1, -1, -1, -1};
  for (int x = tid; x < NBK / 4; x += kResolveThreads) ((i32x4*)Hn)[x] = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (i0 + j < k) e_hit[i0 + j] = INT_MAX;
  PHASE_POINT(1);
  // Barriers below order LDS only: no thread reads global memory that another
  // thread of the workgroup wrote, so the slot-state loads stay in flight
  // through step 1 and the row-ID and stamp stores never hold a barrier.
  lds_barrier();

  // Step 1: validity, resident pages, table of pending positions.  A
  // thread's inserts issue their fill-count adds together.
  int n_res = 0, n_trip = 0;
  unsigned pend = 0;
  uint32_t ibk[KPT];
  int icell[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = i0 + j;
    if (i >= k) continue;
    const int t = tr[j];
    if (t < 0 || (int64_t)t >= n) {
      outb[i] = -1;
      continue;
    }
    if constexpr (PAGED) {
      const int pg = pgs[j];
      if (pg >= 0 && (int64_t)pg < p.resident_pages) {
        const int off = p.P_shift >= 0 ? (t & (p.P - 1)) : t % p.P;
        outb[i] = (int)((int64_t)p.R * S + (int64_t)pg * p.P + off);
        ++n_res;
        continue;
      }
      if (pg >= 0) ++n_trip;
    }
    pend |= 1u << j;
    e_tok[i] = t;
    ibk[j] = hash_pos(t, bshift);
    icell[j] = atomicAdd(&Hn[ibk[j]], vone);
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (!((pend >> j) & 1u)) continue;
    // a full bucket: the next one (the table has at least twice as many
    // cells as entries, so a bucket with room is always reached)
    while (icell[j] >= kBucketCells) {
      ibk[j] = (ibk[j] + 1) & (NBK - 1);
      icell[j] = atomicAdd(&Hn[ibk[j]], vone);
    }
    const int cell = (int)ibk[j] * kBucketCells + icell[j];
    Hc[cell] = tr[j];
    Hi[cell] = (uint16_t)(i0 + j);
  }
  PHASE_POINT(2);
  lds_barrier();

  // Step 2: probe the table with every slot's token; the SPT probes of a
  // thread advance together (their first buckets read back to back), so a
  // wavefront waits for its longest chain once.  A position is in the table
  // once per pending entry that holds it, so at most one cell matches unless
  // the row repeats a position (outside the contract): then the matched cell
  // may be wrong, and the index check below keeps every access in range.
  int hidx[SPT];  // top-k index of the pending entry this slot's token matches, or -1
  {
    constexpr int BV = kBucketCells / 4;  // 16-byte reads per bucket
    static_assert(kBucketCells == 4 || kBucketCells == 8, "bucket reads");
    uint32_t g[SPT];
    i32x4 v[SPT][BV];
    int hcell[SPT];  // table cell holding this slot's token, or -1
    unsigned live = 0;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int tok = sr[j];
      if ((s0 + j < S) && tok >= 0 && (int64_t)tok < n) live |= 1u << j;
      g[j] = hash_pos(tok, bshift);  // in range for any token
#pragma unroll
      for (int e = 0; e < BV; ++e) v[j][e] = ((const i32x4*)Hc)[BV * g[j] + e];
      hcell[j] = -1;
    }
    while (true) {
      unsigned next = 0;
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const int tok = sr[j];
        const bool m0 = v[j][0].x == tok, m1 = v[j][0].y == tok, m2 = v[j][0].z == tok, m3 = v[j][0].w == tok;
        bool any = m0 | m1 | m2 | m3;
        int q = ((m1 | m3) ? 1 : 0) | ((m2 | m3) ? 2 : 0);
        if constexpr (BV == 2) {
          const bool m4 = v[j][1].x == tok, m5 = v[j][1].y == tok, m6 = v[j][1].z == tok, m7 = v[j][1].w == tok;
          any = any | m4 | m5 | m6 | m7;
          q = ((m1 | m3 | m5 | m7) ? 1 : 0) | ((m2 | m3 | m6 | m7) ? 2 : 0) | ((m4 | m5 | m6 | m7) ? 4 : 0);
        }
        const bool lj = (live >> j) & 1u;
        hcell[j] = (lj && any) ? (int)(kBucketCells * g[j]) + q : hcell[j];
        // a full bucket without a match: the next one
        next |= (lj && !any && v[j][BV - 1].w != -1) ? 1u << j : 0u;
      }
      if (next == 0) break;
      live = next;
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const bool nj = (next >> j) & 1u;
        g[j] = nj ? (g[j] + 1) & (NBK - 1) : g[j];
#pragma unroll
        for (int e = 0; e < BV; ++e) v[j][e] = ((const i32x4*)Hc)[BV * g[j] + e];
      }
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int x = hcell[j] >= 0 ? (int)Hi[hcell[j] >= 0 ? hcell[j] : 0] : -1;
      hidx[j] = x < k ? x : -1;
    }
#pragma unroll
    for (int j = 0; j < SPT; ++j)
      if (hidx[j] >= 0) atomicMin(&e_hit[hidx[j]], s0 + j);
  }
  PHASE_POINT(3);
  lds_barrier();

  // Step 3: hits and misses.  An entry's hit slot is the one its e_hit
  // names; a miss's host row is loaded as soon as the miss is known and used
  // only at the end (every lane loads, hits and invalid entries the row's
  // first location, so the load sits in no branch that would wait for it).
  // A slot is a hit slot if the entry its token matched names it.  Then the per-wave partials: counters, misses, and the
  // smallest victim key (occupied << 32 | biased stamp) among the
  // candidates (slots that are not hit slots); and the ranking bitmaps of
  // the first window are cleared (the table is dead).
  const int64_t* locr = p.locs + (int64_t)r * p.max_seq_len;
  int n_hit = 0, my_miss = 0;
  unsigned missbits = 0;
  int sh[KPT];
  unsigned hitbits = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    sh[j] = k > 0 ? e_hit[min(i0 + j, k - 1)] : INT_MAX;
    const unsigned pj = (pend >> j) & 1u;
    const unsigned mj = pj & (sh[j] == INT_MAX ? 1u : 0u);
    missbits |= mj << j;
    hitbits |= (pj & (mj ^ 1u)) << j;
    my_miss += (int)mj;
  }
  n_hit = __popc(hitbits);
  // The misses' host rows: one unconditional load per entry (the row's first
  // location for the others), so no branch joins wait for them.
  int64_t hraw[KPT];  // host row of each miss (entries that are not misses: unused)
#pragma unroll
  for (int j = 0; j < KPT; ++j) hraw[j] = locr[tr[j] & -(int)((missbits >> j) & 1u)];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (hitbits & (1u << j)) outb[i0 + j] = rowbase + sh[j];  // the slot's owner refreshes its stamp
  unsigned hitm = 0;
#pragma unroll
  for (int j = 0; j < SPT; ++j)
    if (hidx[j] >= 0 && e_hit[hidx[j]] == s0 + j) hitm |= 1u << j;
  uint64_t key[SPT];
  unsigned cand = 0;
  uint64_t kmine = ~0ull;
#pragma unroll
  for (int j = 0; j < SPT; ++j) {
    key[j] = ((uint64_t)(sr[j] >= 0 ? 1u : 0u) << 32) | (uint64_t)((uint32_t)lr[j] ^ 0x80000000u);
    if (s0 + j < S && !(hitm & (1u << j))) {
      cand |= 1u << j;
      kmine = key[j] < kmine ? key[j] : kmine;
    }
  }
  int mpre;  // misses in lower lanes of this wavefront
  // This thread's candidates holding the wavefront's smallest key, and how
  // many such candidates lower lanes hold: if the row's smallest key covers
  // every miss, they give the ranks with no window at all.
  unsigned at0w = 0;
  uint64_t kmw;
  {
    const int a0 = wave_sum_small<bits_for(KPT)>(n_hit);
    const int a1 = wave_sum_small<bits_for(KPT)>(n_res);
    const int a2 = wave_sum_small<bits_for(KPT)>(n_trip);
    int wt = 0;
    mpre = 0;
#pragma unroll
    for (int q = 0; q < bits_for(KPT); ++q) {
      const uint64_t m = __ballot((my_miss >> q) & 1);
      mpre += lane_prefix(m) << q;
      wt += __popcll(m) << q;
    }
    const uint64_t km = wave_min_key(kmine);
    kmw = km;
#pragma unroll
    for (int j = 0; j < SPT; ++j) at0w |= (((cand >> j) & 1u) && key[j] == km ? 1u : 0u) << j;
    const int wt0 = wave_sum_small<bits_for(SPT)>(__popc(at0w));
    if (lane == 0) {
      scr[kScrStats + wid] = a0;
      scr[kScrStats + 16 + wid] = a1;
      scr[kScrStats + 32 + wid] = a2;
      scr[kScrMiss + wid] = wt;
      scr[kScrKey0 + wid] = wt0;
      ((uint64_t*)(scr + kScrMin))[wid] = km;
    }
  }
  // Ranking bitmaps [word][key] with a padded (odd) key stride, so that the
  // lanes of one word, whose slots carry different keys, reach different
  // LDS banks: bit s % 64 of word s / 64 of key d = slot s has key base + d.
  const int NBIN = L.bins, W = L.words, BST = L.bins + 1;
  uint64_t* bm = (uint64_t*)(smem + L.off_bits);    // [W][BST] slots of each key in the window
  uint32_t* wpre = (uint32_t*)(smem + L.off_wpre);  // [W][BST] set bits of the key in earlier words
  for (int x = tid; x < W * BST; x += kResolveThreads) bm[x] = 0ull;
  PHASE_POINT(4);
  lds_barrier();

  // Step 4: the ordered miss list (ascending top-k index), and the misses'
  // count m; then victims, in (occupied, stamp, slot) order among the
  // candidates.  A window takes the keys base .. base + NBIN - 1 above the
  // smallest remaining key: each key's candidates set their bits in that
  // key's slot bitmap, each bitmap's words get exclusive popcount prefixes,
  // and a candidate's rank is (victims so far) + (candidates of smaller keys
  // in the window) + (candidates of its key at lower slots): the exact
  // position in key-then-slot order, with three barriers per window.
  // Keys spread over more than kMaxRankWindows windows fall back to a
  // bitonic sort of the remaining candidates.
  int m_total, mpos;
  {
    const uint32_t inc = wave_inclusive_sum(lane < kResolveWaves ? (uint32_t)scr[kScrMiss + lane] : 0u);
    m_total = __builtin_amdgcn_readlane((int)inc, 63);
    mpos = (wid > 0 ? __builtin_amdgcn_readlane((int)inc, wid - 1) : 0) + mpre;
  }
  const int mpos0 = mpos;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (missbits & (1u << j)) m_entry[mpos++] = i0 + j;
  int64_t* psrc = p.plan_src + (int64_t)b * p.plan_stride;
  // The misses' host rows as the fused copy keeps them (see host_row32),
  // converted for every entry outside any branch, and used by an empty asm
  // statement: the wait for the host-row loads then sits here on every path,
  // before the copy's first loads below, and nothing later waits on the
  // in-order vector-memory counter behind those loads.
  int32_t h32[KPT];
  if constexpr (COPY) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      h32[j] = host_row32(hraw[j]);
      asm volatile("" : : "v"(h32[j]));
    }
    int mp = mpos0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (missbits & (1u << j)) m_h[mp++] = h32[j];
  }

  int vr[SPT];  // rank of this slot among the victims, or -1
#pragma unroll
  for (int j = 0; j < SPT; ++j) vr[j] = -1;
  int need = m_total, vbase = 0;
  constexpr int RIF = kCopyRowsInFlight;
  u32x4 pre[RIF];
  bool have_pre = false;
  // Fused copy, first rows: once the miss list is visible, each wavefront
  // loads its first kCopyRowsInFlight rows of the first layer, so the host
  // link works while the victims are ranked and the plan is written; the
  // rows are stored once their slots are known.  (m_total is uniform.)
  if (COPY && m_total > 0 && p.units <= kWave) {
    lds_barrier();
    have_pre = true;
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
  const int wrd = s0 >> 6, bit0 = s0 & 63;  // this thread's slots share one bitmap word
#ifdef HISPARSE_PHASE_TRACE
  int trace_windows = 0;
#endif
  uint64_t base0 = 0;  // the row's smallest key (the first window's base)
  if (need > 0) {
    // The row's smallest key: if its candidates cover every miss, their
    // slot order is the victim order (no window, no bitmap).  Waves whose
    // own smallest key is larger hold none of them.  (Uniform decision.)
    const uint64_t kp = lane < kResolveWaves ? ((const uint64_t*)(scr + kScrMin))[lane] : ~0ull;
    const uint64_t base = wave_min_key(kp);
    base0 = base;
    const uint32_t inc = wave_inclusive_sum(
        lane < kResolveWaves && kp == base ? (uint32_t)scr[kScrKey0 + lane] : 0u);
    if (__builtin_amdgcn_readlane((int)inc, 63) >= need) {
      if (kmw == base) {
        const int c0 = __popc(at0w);
        int rk = wid > 0 ? __builtin_amdgcn_readlane((int)inc, wid - 1) : 0;
#pragma unroll
        for (int q = 0; q < bits_for(SPT); ++q) rk += lane_prefix(__ballot((c0 >> q) & 1)) << q;
#pragma unroll
        for (int j = 0; j < SPT; ++j)
          if (at0w & (1u << j)) {
            if (rk < need) vr[j] = rk;
            ++rk;
          }
      }
      vbase = need;
      need = 0;
    }
  }
  if (NBIN > 0 && need > 0) {
#pragma unroll 1
    for (int win = 0;; ++win) {
#ifdef HISPARSE_PHASE_TRACE
      trace_windows = win + 1;
#endif
      const uint64_t* kmin_part = (const uint64_t*)(scr + kScrMin) + 16 * (win & 1);
      // the other half holds the next window's minima only after two more
      // barriers; until then it takes this window's per-wave counts below
      int* key0_part = scr + kScrMin + 32 * ((win + 1) & 1);
      // (the first window's base and smallest-key test were done above)
      const uint64_t base = win == 0 ? base0 : wave_min_key(lane < kResolveWaves ? kmin_part[lane] : ~0ull);
      unsigned inwin = 0, at0 = 0;
      int dd[SPT];
#pragma unroll
      for (int j = 0; j < SPT; ++j) {
        const uint64_t d = key[j] - base;
        dd[j] = (int)d;
        if ((cand & (1u << j)) && d < (uint64_t)NBIN) {
          inwin |= 1u << j;
          at0 |= (d == 0 ? 1u : 0u) << j;
          atomicOr((unsigned long long*)&bm[wrd * BST + dd[j]], 1ull << (bit0 + j));
        }
      }
      // Candidates of the smallest key, counted per wavefront on the way: if
      // they cover every remaining miss, their slot-order prefix is the rank
      // and the window needs no word prefixes (a few misses, as on steps
      // with high reuse).
      int pre0 = 0;
      if (win > 0) {
        const int c0 = __popc(at0);
        int wt = 0;
#pragma unroll
        for (int q = 0; q < bits_for(SPT); ++q) {
          const uint64_t m = __ballot((c0 >> q) & 1);
          pre0 += lane_prefix(m) << q;
          wt += __popcll(m) << q;
        }
        if (lane == 0) key0_part[wid] = wt;
      }
      lds_barrier();
      if (win > 0) {
        const uint32_t k0 = lane < kResolveWaves ? (uint32_t)key0_part[lane] : 0u;
        const uint32_t inc0 = wave_inclusive_sum(k0);
        const int tot0 = __builtin_amdgcn_readlane((int)inc0, 63);
        if (tot0 >= need) {  // workgroup-uniform
          int rk = (wid > 0 ? __builtin_amdgcn_readlane((int)inc0, wid - 1) : 0) + pre0;
#pragma unroll
          for (int j = 0; j < SPT; ++j)
            if (at0 & (1u << j)) {
              if (rk < need) vr[j] = vbase + rk;
              ++rk;
            }
          vbase += need;
          need = 0;
          break;
        }
      }
      // Word prefixes of each key's bitmap (wavefront wid takes keys wid,
      // wid + 16) and the number of candidates of each key.
      for (int bin = wid; bin < NBIN; bin += kResolveWaves) {
        uint32_t carry = 0;
        for (int w0 = 0; w0 < W; w0 += kWave) {
          const int w = w0 + lane;
          const uint32_t pc = w < W ? (uint32_t)__popcll(bm[w * BST + bin]) : 0u;
          const uint32_t inc = wave_inclusive_sum(pc);
          if (w < W) wpre[w * BST + bin] = carry + inc - pc;
          carry += (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
        }
        if (lane == 0) scr[kScrBtot + bin] = (int)carry;
      }
      lds_barrier();
      const uint32_t bcnt = lane < NBIN ? (uint32_t)scr[kScrBtot + lane] : 0u;
      const uint32_t binc = wave_inclusive_sum(bcnt);
      const int tot = __builtin_amdgcn_readlane((int)binc, 63);
      const int cexcl = (int)(binc - bcnt);  // lane d: candidates of keys below base + d
      // Every slot's three LDS reads are issued before any is used (a slot
      // outside the window reads key 0's and ignores it), four slots at a time.
      constexpr int RC = SPT < 4 ? SPT : 4;
#pragma unroll
      for (int j0 = 0; j0 < SPT; j0 += RC) {
        int below[RC], wp[RC];
        uint64_t word[RC];
#pragma unroll
        for (int c = 0; c < RC; ++c) {
          const int j = j0 + c;
          const int d = (inwin & (1u << j)) ? dd[j] : 0;
          below[c] = __shfl(cexcl, d, kWave);
          word[c] = bm[wrd * BST + d];
          wp[c] = (int)wpre[wrd * BST + d];
        }
#pragma unroll
        for (int c = 0; c < RC; ++c) {
          const int j = j0 + c;
          const int rank = below[c] + wp[c] + __popcll(word[c] & ((1ull << (bit0 + j)) - 1ull));
          if ((inwin & (1u << j)) && rank < need) vr[j] = vbase + rank;
        }
      }
      cand &= ~inwin;
      const int take = tot < need ? tot : need;
      vbase += take;
      need -= take;
      if (need == 0 || win + 1 == kMaxRankWindows) break;
      // Next window: the smallest key left, once every thread is done
      // reading the bitmaps.
      lds_barrier();
      for (int x = tid; x < W * BST; x += kResolveThreads) bm[x] = 0ull;
      uint64_t km = ~0ull;
#pragma unroll
      for (int j = 0; j < SPT; ++j)
        if ((cand & (1u << j)) && key[j] < km) km = key[j];
      km = wave_min_key(km);
      if (lane == 0) ((uint64_t*)(scr + kScrMin))[16 * ((win + 1) & 1) + wid] = km;
      lds_barrier();
    }
  }
#ifdef HISPARSE_PHASE_TRACE
  PHASE_INFO(trace_windows, need > 0 ? 1 : 0);
#endif
  if (need > 0) {  // keys spread over many windows: sort the remaining candidates
    const int N = L.sort_size;
    lds_barrier();  // the table and bitmap regions are reused for the sort
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
    lds_barrier();  // the victim list is rewritten below
  }

  PHASE_POINT(5);
  // Step 5: the victim of rank j takes the j-th miss: its owner sets token,
  // row ID and the device row of plan entry j; the miss's owner writes the
  // host row of plan entry j.  The fused copy keeps the plan's device rows
  // in the victim list (its host rows are the miss list's).  Then every
  // thread writes its slot run back once: stamps of hit and victim slots,
  // tokens of victim slots (vector stores, not one scattered store per slot).
  int32_t* pdst = p.plan_dst + (int64_t)b * p.plan_stride;
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
    pdst[v] = row;
    if (COPY) victim[v] = row;
  }
  {
    // The plan's host rows.  The fused instance stores the 32-bit values of
    // its copy list (a row outside [0, 2^31) as -1, out of range for every
    // pool either way), which wait for no load.
    int mp = mpos0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (missbits & (1u << j)) psrc[mp++] = COPY ? (int64_t)h32[j] : hraw[j];
  }
  const int32_t c = (int32_t)((uint32_t)clk_now + 1u);
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
  PHASE_POINT(6);

  // Fused miss copy: one wavefront per (layer, miss) row, lane l carrying
  // 16-byte unit l, kCopyRowsInFlight rows per wavefront and iteration.  The
  // compiler issues an iteration's loads one after another (each waits for
  // the one before, through the choice of the row loaded ahead), so about one
  // row per wavefront is in flight; measured, that is faster over the host
  // link than three in flight (135.3 against 133.9 us per DSA-decode step)
  // and than 8 or 4 copying wavefronts per workgroup (138.4, 136.3 us).  Row
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
      bool dok[RIF];
#pragma unroll
      for (int q = 0; q < RIF; ++q) {
        const bool real = u + q * kResolveWaves < total;
        const int uq = real ? u + q * kResolveWaves : u;
        const int l = uq / m_total, j = uq - l * m_total;
        const int64_t h = __builtin_amdgcn_readfirstlane(m_h[j]);   // -1: outside [0, 2^31)
        const int d = __builtin_amdgcn_readfirstlane(victim[j]);    // the plan's device row
        const bool ok = h >= 0 && h < p.host_rows[l];
        // every miss's row is one of this request's hot rows; the check keeps
        // a store inside them whatever the list holds
        dok[q] = d >= rowbase && d < rowbase + S;
        src[q] = ok ? (const gu4*)p.host_pool[l] + h * U : (const gu4*)p.zero_row;
        dst[q] = (gu4*)p.dev_pool[l] + (int64_t)(dok[q] ? d : rowbase) * U;
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
        for (int q = 0; q < RIF; ++q)
          if (dok[q]) dst[q][part] = v[q];
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
  PHASE_POINT(7);
}

template <int SPT, int KPT, bool PAGED>
void launch_p(const ResolveParams& p, int batch, size_t lds, hipStream_t stream) {
  const dim3 g(batch), t(kResolveThreads);
  if (p.copy_layers > 0) {
    if (p.vec_state) hipLaunchKernelGGL((resolve_kernel<SPT, KPT, true, true, PAGED>), g, t, lds, stream, p);
    else hipLaunchKernelGGL((resolve_kernel<SPT, KPT, true, false, PAGED>), g, t, lds, stream, p);
  } else {
    if (p.vec_state) hipLaunchKernelGGL((resolve_kernel<SPT, KPT, false, true, PAGED>), g, t, lds, stream, p);
    else hipLaunchKernelGGL((resolve_kernel<SPT, KPT, false, false, PAGED>), g, t, lds, stream, p);
  }
}

template <int SPT, int KPT>
hipError_t launch_t(const ResolveParams& p, int batch, size_t lds, hipStream_t stream) {
  if (p.bt != nullptr) launch_p<SPT, KPT, true>(p, batch, lds, stream);
  else launch_p<SPT, KPT, false>(p, batch, lds, stream);
  return hipGetLastError();
}

template <int SPT>
hipError_t launch_k(const ResolveParams& p, int batch, size_t lds, hipStream_t stream, int kpt) {
  switch (kpt) {
    case 1: return launch_t<SPT, 1>(p, batch, lds, stream);
    case 2: return launch_t<SPT, 2>(p, batch, lds, stream);
    default: return launch_t<SPT, 4>(p, batch, lds, stream);  // kMaxEntriesPerThread
  }
}

template <int SPT, int KPT>
hipError_t set_attr() {
  const void* fns[8] = {(const void*)resolve_kernel<SPT, KPT, false, false, false>,
                        (const void*)resolve_kernel<SPT, KPT, false, true, false>,
                        (const void*)resolve_kernel<SPT, KPT, true, false, false>,
                        (const void*)resolve_kernel<SPT, KPT, true, true, false>,
                        (const void*)resolve_kernel<SPT, KPT, false, false, true>,
                        (const void*)resolve_kernel<SPT, KPT, false, true, true>,
                        (const void*)resolve_kernel<SPT, KPT, true, false, true>,
                        (const void*)resolve_kernel<SPT, KPT, true, true, true>};
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
  return e;
}

}  // namespace

hipError_t launch_resolve(ResolveParams p, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  p.lds = resolve_lds_layout(p.S, p.k);
  p.P_shift = (p.P > 0 && (p.P & (p.P - 1)) == 0) ? ilog2(p.P) : -1;
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

#ifdef HISPARSE_PHASE_TRACE
hipError_t phase_trace_clear() {
  void* d = nullptr;
  hipError_t e = hipGetSymbolAddress(&d, HIP_SYMBOL(g_phase_trace));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemset(d, 0, sizeof(g_phase_trace));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  return e;
}

hipError_t phase_trace_read(uint64_t* host, size_t count) {
  if (count * sizeof(uint64_t) != sizeof(g_phase_trace)) return hipErrorInvalidValue;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(host, HIP_SYMBOL(g_phase_trace), sizeof(g_phase_trace));
  return e;
}
#endif

hipError_t prepare_resolve(size_t) {
  hipError_t e = set_attr_k<1>();
  if (e == hipSuccess) e = set_attr_k<2>();
  if (e == hipSuccess) e = set_attr_k<4>();
  if (e == hipSuccess) e = set_attr_k<8>();
  if (e == hipSuccess) e = set_attr_k<16>();
  return e;
}

}  // namespace hisparse
