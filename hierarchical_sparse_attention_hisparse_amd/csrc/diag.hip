// diag.hip -- entry points of the diagnostic library (libhisparse_diag.so):
// the plan kernel's phase trace, read out, and floor kernels of the plan
// kernel's launch shape (one 1024-thread workgroup per batch row), which
// price the launch, its dependent global round trips and its memory chain
// without the computation between them.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "../../include/hisparse.h"
#include "../../include/hisparse_diag.h"
#include "common.h"
#include "kernels.h"

static_assert(HISPARSE_TRACE_ROWS == hisparse::kTraceRows, "trace rows");
static_assert(HISPARSE_TRACE_WAVES == hisparse::kResolveWaves, "trace waves");
static_assert(HISPARSE_TRACE_POINTS == hisparse::kTracePoints, "trace points");

namespace hisparse {
namespace {

constexpr int kFloorThreads = kResolveThreads;
constexpr int kFloorMaxK = 4096;  // entries per row: at most 4 per thread

struct FloorParams {
  int32_t k, S, R;
  int64_t max_seq_len;
  const int32_t* req;
  const int32_t* topk;
  const int32_t* st;
  const int32_t* lru;
  const int64_t* locs;
  int32_t* out;
};

__device__ inline int clamp_req(int r, int R) { return r < 0 ? 0 : (r >= R ? R - 1 : r); }

__global__ __launch_bounds__(kFloorThreads) void floor_empty_kernel() {}

// One round trip: the request row, stored to the row's outputs.
__global__ __launch_bounds__(kFloorThreads) void floor_one_kernel(FloorParams p) {
  const int b = blockIdx.x;
  const int r = p.req[b];
  for (int i = threadIdx.x; i < p.k; i += kFloorThreads) p.out[(int64_t)b * p.k + i] = r;
}

// Two dependent round trips: the request row, then its slot map and stamps
// (coalesced), folded per thread and stored.
__global__ __launch_bounds__(kFloorThreads) void floor_two_kernel(FloorParams p) {
  const int b = blockIdx.x;
  const int r = clamp_req(p.req[b], p.R);
  const int32_t* st = p.st + (int64_t)r * p.S;
  const int32_t* lru = p.lru + (int64_t)r * p.S;
  int acc = 0;
  for (int s = threadIdx.x; s < p.S; s += kFloorThreads) acc += st[s] ^ lru[s];
  for (int i = threadIdx.x; i < p.k; i += kFloorThreads) p.out[(int64_t)b * p.k + i] = acc;
}

// The plan's memory chain: top-k row and request row; slot map and stamps;
// a workgroup exchange; one host location per entry, whose address depends
// on the exchanged slot data (as a miss's does); row IDs stored.
__global__ __launch_bounds__(kFloorThreads) void floor_chain_kernel(FloorParams p) {
  __shared__ int part[kFloorThreads / kWave];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & (kWave - 1), wid = tid / kWave;
  int t[kFloorMaxK / kFloorThreads];
#pragma unroll
  for (int j = 0; j < kFloorMaxK / kFloorThreads; ++j) {
    const int i = tid + j * kFloorThreads;
    t[j] = i < p.k ? p.topk[(int64_t)b * p.k + i] : 0;
  }
  const int r = clamp_req(p.req[b], p.R);
  const int32_t* st = p.st + (int64_t)r * p.S;
  const int32_t* lru = p.lru + (int64_t)r * p.S;
  int acc = 0;
  for (int s = tid; s < p.S; s += kFloorThreads) acc += st[s] ^ lru[s];
  for (int o = kWave / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (lane == 0) part[wid] = acc;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int w = 0; w < kFloorThreads / kWave; ++w) tot += part[w];
  const int64_t* locr = p.locs + (int64_t)r * p.max_seq_len;
#pragma unroll
  for (int j = 0; j < kFloorMaxK / kFloorThreads; ++j) {
    const int i = tid + j * kFloorThreads;
    if (i < p.k) {
      int64_t pos = t[j] < 0 ? 0 : (t[j] >= p.max_seq_len ? p.max_seq_len - 1 : t[j]);
      pos = tot == INT_MIN ? 0 : pos;  // the address waits for the slot data
      p.out[(int64_t)b * p.k + i] = (int32_t)locr[pos];
    }
  }
}

// Hit detection alone, both ways round, one 1024-thread workgroup per batch
// row: out[b][i] = the lowest slot of the request holding entry i's
// position, or -1.
//   MODE 0: the entries' positions go into the table (top-k index per cell)
//           and every slot probes it with its token (the library's way);
//   MODE 1: the slots' tokens go into the table (lowest slot per cell) and
//           every entry probes it with its position (a slot -> token map).
// Modes 0 and 1 use single-cell linear probing with 4 cells per inserted
// item.  Modes 2 and 3 are the same two directions with the resolver's kind
// of table: buckets of 4 cells handed out in order by a fill count per
// bucket (one atomic add per insert, the next bucket past a full one) and
// read 16 bytes at a time; mode 2 has 8 cells per entry, as the resolver
// does (4 at k = 4096), mode 3 4 cells per slot (8 would take 256 KB of
// LDS at S = 4096).
constexpr int kHitMaxK = 4096, kHitMaxS = 4096;

__device__ inline uint32_t hit_hash(int t, int shift) { return ((uint32_t)t * 2654435761u) >> shift; }

struct HitParams {
  int32_t k, S, R;
  int64_t max_seq_len;
  const int32_t* req;
  const int32_t* topk;
  const int32_t* seq;
  const int32_t* st;
  int32_t* out;
  int32_t cells, shift;  // table cells (power of two) and hash shift (modes 2, 3: of the buckets)
};

typedef int hit_i32x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(kFloorThreads) void hit_detect_kernel(HitParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* key = (int32_t*)smem;           // [cells]: position / token, -1 = free
  int32_t* val = key + p.cells;            // [cells]: MODE 0 top-k index, MODE 1 lowest slot
  int32_t* ehit = val + p.cells;           // MODES 0, 2: [k] lowest hit slot per entry
  int32_t* cnt = ehit + (MODE == 2 ? p.k : 0);  // MODES 2, 3: [cells / 4] fill count per bucket
  const int nbk = p.cells / 4;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int r = clamp_req(p.req[b], p.R);
  const int64_t n = p.seq[b] < p.max_seq_len ? (int64_t)p.seq[b] : p.max_seq_len;
  const int32_t* tk = p.topk + (int64_t)b * p.k;
  const int32_t* st = p.st + (int64_t)r * p.S;
  const int mask = p.cells - 1;
  for (int x = tid; x < p.cells; x += kFloorThreads) {
    key[x] = -1;
    val[x] = INT_MAX;
  }
  if (MODE == 0 || MODE == 2)
    for (int i = tid; i < p.k; i += kFloorThreads) ehit[i] = INT_MAX;
  if (MODE >= 2)
    for (int x = tid; x < nbk; x += kFloorThreads) cnt[x] = 0;
  __syncthreads();
  // A bucketed insert: the cell the bucket's fill count names, past full
  // buckets (the table has at least twice as many cells as items).
  auto bucket_insert = [&](int t, int v) {
    uint32_t bk = hit_hash(t, p.shift);
    int c = atomicAdd(&cnt[bk], 1);
    while (c >= 4) {
      bk = (bk + 1) & (uint32_t)(nbk - 1);
      c = atomicAdd(&cnt[bk], 1);
    }
    key[4 * bk + c] = t;
    val[4 * bk + c] = v;
  };
  if (MODE == 2) {
    for (int i = tid; i < p.k; i += kFloorThreads) {
      const int t = tk[i];
      if (t < 0 || (int64_t)t >= n) continue;
      bucket_insert(t, i);
    }
    __syncthreads();
    for (int s = tid; s < p.S; s += kFloorThreads) {
      const int tok = st[s];
      if (tok < 0 || (int64_t)tok >= n) continue;
      for (uint32_t bk = hit_hash(tok, p.shift);; bk = (bk + 1) & (uint32_t)(nbk - 1)) {
        const hit_i32x4 v = ((const hit_i32x4*)key)[bk];  // positions are distinct: one match at most
        const int q = v.x == tok ? 0 : v.y == tok ? 1 : v.z == tok ? 2 : v.w == tok ? 3 : -1;
        if (q >= 0) {
          atomicMin(&ehit[val[4 * bk + q]], s);
          break;
        }
        if (v.w == -1) break;  // a bucket with room ends the chain
      }
    }
    __syncthreads();
    for (int i = tid; i < p.k; i += kFloorThreads)
      p.out[(int64_t)b * p.k + i] = ehit[i] == INT_MAX ? -1 : ehit[i];
  } else if (MODE == 3) {
    for (int s = tid; s < p.S; s += kFloorThreads) {
      const int tok = st[s];
      if (tok < 0 || (int64_t)tok >= n) continue;
      bucket_insert(tok, s);
    }
    __syncthreads();
    for (int i = tid; i < p.k; i += kFloorThreads) {
      const int t = tk[i];
      int res = INT_MAX;
      if (t >= 0 && (int64_t)t < n) {
        // A token held by several slots sits in several cells, all on its
        // chain up to the first bucket with room: the lowest slot of them.
        for (uint32_t bk = hit_hash(t, p.shift);; bk = (bk + 1) & (uint32_t)(nbk - 1)) {
          const hit_i32x4 v = ((const hit_i32x4*)key)[bk];
          if (v.x == t) res = min(res, val[4 * bk]);
          if (v.y == t) res = min(res, val[4 * bk + 1]);
          if (v.z == t) res = min(res, val[4 * bk + 2]);
          if (v.w == t) res = min(res, val[4 * bk + 3]);
          if (v.w == -1) break;
        }
      }
      p.out[(int64_t)b * p.k + i] = res == INT_MAX ? -1 : res;
    }
  } else if (MODE == 0) {
    for (int i = tid; i < p.k; i += kFloorThreads) {
      const int t = tk[i];
      if (t < 0 || (int64_t)t >= n) continue;
      uint32_t h = hit_hash(t, p.shift);
      while (true) {
        const int prev = atomicCAS(&key[h], -1, t);
        if (prev == -1) {
          val[h] = i;
          break;
        }
        if (prev == t) break;
        h = (h + 1) & mask;
      }
    }
    __syncthreads();
    for (int s = tid; s < p.S; s += kFloorThreads) {
      const int tok = st[s];
      if (tok < 0 || (int64_t)tok >= n) continue;
      for (uint32_t h = hit_hash(tok, p.shift);; h = (h + 1) & mask) {
        const int c = key[h];
        if (c == tok) {
          atomicMin(&ehit[val[h]], s);
          break;
        }
        if (c == -1) break;
      }
    }
    __syncthreads();
    for (int i = tid; i < p.k; i += kFloorThreads)
      p.out[(int64_t)b * p.k + i] = ehit[i] == INT_MAX ? -1 : ehit[i];
  } else {
    for (int s = tid; s < p.S; s += kFloorThreads) {
      const int tok = st[s];
      if (tok < 0 || (int64_t)tok >= n) continue;
      for (uint32_t h = hit_hash(tok, p.shift);; h = (h + 1) & mask) {
        const int prev = atomicCAS(&key[h], -1, tok);
        if (prev == -1 || prev == tok) {
          atomicMin(&val[h], s);
          break;
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < p.k; i += kFloorThreads) {
      const int t = tk[i];
      int res = -1;
      if (t >= 0 && (int64_t)t < n) {
        for (uint32_t h = hit_hash(t, p.shift);; h = (h + 1) & mask) {
          const int c = key[h];
          if (c == t) {
            res = val[h];
            break;
          }
          if (c == -1) break;
        }
      }
      p.out[(int64_t)b * p.k + i] = res;
    }
  }
}

// Last-arriver exchange among `groups` workgroups of one batch row: partials
// written and fenced, the row's counter bumped; the last workgroup reads
// every partial and resets the counter.  No workgroup waits for another.
constexpr int kExchangeThreads = 256;
constexpr int kExchangeMaxGroups = 16;
static_assert(HISPARSE_EXCHANGE_ROW_INTS == 64 + 64 * kExchangeMaxGroups, "exchange row");

__global__ __launch_bounds__(kExchangeThreads) void exchange_kernel(int32_t* scratch, int groups) {
  __shared__ int last;
  const int b = blockIdx.x / groups, g = blockIdx.x - b * groups;
  const int tid = threadIdx.x;
  int32_t* row = scratch + (int64_t)b * HISPARSE_EXCHANGE_ROW_INTS;
  if (tid < 64) row[64 + g * 64 + tid] = g + tid;
  __threadfence();
  __syncthreads();
  if (tid == 0) last = atomicAdd(&row[0], 1) == groups - 1 ? 1 : 0;
  __syncthreads();
  if (!last) return;
  __threadfence();
  int s = 0;
  for (int x = tid; x < groups * 64; x += kExchangeThreads)
    s += __hip_atomic_load(&row[64 + x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid < 32) row[32 + tid] = s;
  if (tid == 0) row[0] = 0;
}

}  // namespace
}  // namespace hisparse

using namespace hisparse;

extern "C" {

int hisparse_diag_phase_clear(void) {
  const hipError_t e = phase_trace_clear();
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return report_error(HISPARSE_EHIP, "phase trace clear: %s", hipGetErrorString(e));
  }
  return HISPARSE_OK;
}

int hisparse_diag_phase_read(uint64_t* host_out, size_t count) {
  if (!host_out) return report_error(HISPARSE_EINVAL, "host_out is NULL");
  if (count != (size_t)HISPARSE_TRACE_WORDS)
    return report_error(HISPARSE_EINVAL, "count %zu != %d", count, HISPARSE_TRACE_WORDS);
  const hipError_t e = phase_trace_read(host_out, count);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return report_error(HISPARSE_EHIP, "phase trace read: %s", hipGetErrorString(e));
  }
  return HISPARSE_OK;
}

int hisparse_diag_floor(void* stream, int32_t kind, int32_t batch, int32_t top_k, int32_t slots,
                        int32_t max_requests, int64_t max_seq_len, const int32_t* req_idx,
                        const int32_t* top_k_tokens, const int32_t* slot_tokens,
                        const int32_t* lru_slots, const int64_t* host_cache_locs, int32_t* out,
                        int32_t launches) {
  if (kind < 0 || kind > 3) return report_error(HISPARSE_EINVAL, "kind %d not in [0, 3]", kind);
  if (launches < 1 || launches > (1 << 20))
    return report_error(HISPARSE_EINVAL, "launches %d not in [1, 1048576]", launches);
  if (batch < 1 || batch > 65535) return report_error(HISPARSE_EINVAL, "batch %d not in [1, 65535]", batch);
  if (kind >= 1) {
    if (!req_idx || !out) return report_error(HISPARSE_EINVAL, "req_idx or out is NULL");
    if (top_k < 1 || top_k > kFloorMaxK)
      return report_error(HISPARSE_EINVAL, "top_k %d not in [1, %d]", top_k, kFloorMaxK);
    if (max_requests < 1) return report_error(HISPARSE_EINVAL, "max_requests %d < 1", max_requests);
  }
  if (kind >= 2) {
    if (!slot_tokens || !lru_slots) return report_error(HISPARSE_EINVAL, "slot state is NULL");
    if (slots < 1 || slots > kMaxSlots)
      return report_error(HISPARSE_EINVAL, "slots %d not in [1, %d]", slots, kMaxSlots);
  }
  if (kind == 3) {
    if (!top_k_tokens || !host_cache_locs)
      return report_error(HISPARSE_EINVAL, "top_k_tokens or host_cache_locs is NULL");
    if (max_seq_len < 1) return report_error(HISPARSE_EINVAL, "max_seq_len %lld < 1", (long long)max_seq_len);
  }
  FloorParams p{top_k, slots, max_requests, max_seq_len, req_idx, top_k_tokens,
                slot_tokens, lru_slots, host_cache_locs, out};
  const hipStream_t s = (hipStream_t)stream;
  const dim3 g(batch), t(kFloorThreads);
  for (int n = 0; n < launches; ++n) {
    switch (kind) {
      case 0: hipLaunchKernelGGL(floor_empty_kernel, g, t, 0, s); break;
      case 1: hipLaunchKernelGGL(floor_one_kernel, g, t, 0, s, p); break;
      case 2: hipLaunchKernelGGL(floor_two_kernel, g, t, 0, s, p); break;
      default: hipLaunchKernelGGL(floor_chain_kernel, g, t, 0, s, p); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return report_error(HISPARSE_EHIP, "floor kernel launch: %s", hipGetErrorString(e));
  }
  return HISPARSE_OK;
}

int hisparse_diag_hit_detection(void* stream, int32_t mode, int32_t batch, int32_t top_k, int32_t slots,
                                int32_t max_requests, int64_t max_seq_len, const int32_t* req_idx,
                                const int32_t* top_k_tokens, const int32_t* seq_lens,
                                const int32_t* slot_tokens, int32_t* out, int32_t launches) {
  if (mode < 0 || mode > 3) return report_error(HISPARSE_EINVAL, "mode %d not in [0, 3]", mode);
  if (batch < 1 || batch > 65535) return report_error(HISPARSE_EINVAL, "batch %d not in [1, 65535]", batch);
  if (top_k < 1 || top_k > kHitMaxK)
    return report_error(HISPARSE_EINVAL, "top_k %d not in [1, %d]", top_k, kHitMaxK);
  if (slots < 1 || slots > kHitMaxS)
    return report_error(HISPARSE_EINVAL, "slots %d not in [1, %d]", slots, kHitMaxS);
  if (max_requests < 1 || max_seq_len < 1)
    return report_error(HISPARSE_EINVAL, "max_requests %d or max_seq_len %lld < 1", max_requests,
                        (long long)max_seq_len);
  if (!req_idx || !top_k_tokens || !seq_lens || !slot_tokens || !out)
    return report_error(HISPARSE_EINVAL, "a device array is NULL");
  if (launches < 1 || launches > (1 << 20))
    return report_error(HISPARSE_EINVAL, "launches %d not in [1, 1048576]", launches);
  const int items = (mode == 0 || mode == 2) ? top_k : slots;
  const int per = mode == 2 ? 8 : 4;  // cells per inserted item
  int cells = 64;
  while (cells < per * items) cells <<= 1;
  auto lds_of = [&](int c) {
    return (size_t)2 * c * sizeof(int32_t) + ((mode == 0 || mode == 2) ? (size_t)top_k * sizeof(int32_t) : 0) +
           (mode >= 2 ? (size_t)(c / 4) * sizeof(int32_t) : 0);
  };
  while (lds_of(cells) > kLdsBudget && cells / 2 >= 2 * items) cells >>= 1;  // k = 4096, mode 2: 4 per entry
  const size_t lds = lds_of(cells);
  int lg = 0;
  while ((1 << lg) < (mode >= 2 ? cells / 4 : cells)) ++lg;
  HitParams p{top_k, slots, max_requests, max_seq_len, req_idx, top_k_tokens, seq_lens, slot_tokens,
              out, cells, 32 - lg};
  const void* fns[4] = {(const void*)hit_detect_kernel<0>, (const void*)hit_detect_kernel<1>,
                        (const void*)hit_detect_kernel<2>, (const void*)hit_detect_kernel<3>};
  const void* fn = fns[mode];
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return report_error(HISPARSE_EHIP, "hit detection set-up: %s", hipGetErrorString(e));
  const hipStream_t s = (hipStream_t)stream;
  for (int n = 0; n < launches; ++n) {
    if (mode == 0)
      hipLaunchKernelGGL(hit_detect_kernel<0>, dim3(batch), dim3(kFloorThreads), lds, s, p);
    else if (mode == 1)
      hipLaunchKernelGGL(hit_detect_kernel<1>, dim3(batch), dim3(kFloorThreads), lds, s, p);
    else if (mode == 2)
      hipLaunchKernelGGL(hit_detect_kernel<2>, dim3(batch), dim3(kFloorThreads), lds, s, p);
    else
      hipLaunchKernelGGL(hit_detect_kernel<3>, dim3(batch), dim3(kFloorThreads), lds, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return report_error(HISPARSE_EHIP, "hit detection launch: %s", hipGetErrorString(e));
  }
  return HISPARSE_OK;
}

int hisparse_diag_exchange(void* stream, int32_t batch, int32_t groups, int32_t* scratch,
                           int32_t launches) {
  if (!scratch) return report_error(HISPARSE_EINVAL, "scratch is NULL");
  if (groups < 1 || groups > kExchangeMaxGroups)
    return report_error(HISPARSE_EINVAL, "groups %d not in [1, %d]", groups, kExchangeMaxGroups);
  if (batch < 1 || (int64_t)batch * groups > 65535)
    return report_error(HISPARSE_EINVAL, "batch %d * groups %d not in [1, 65535]", batch, groups);
  if (launches < 1 || launches > (1 << 20))
    return report_error(HISPARSE_EINVAL, "launches %d not in [1, 1048576]", launches);
  const hipStream_t s = (hipStream_t)stream;
  for (int n = 0; n < launches; ++n) {
    hipLaunchKernelGGL(exchange_kernel, dim3(batch * groups), dim3(kExchangeThreads), 0, s, scratch, groups);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return report_error(HISPARSE_EHIP, "exchange kernel launch: %s", hipGetErrorString(e));
  }
  return HISPARSE_OK;
}

}  // extern "C"
