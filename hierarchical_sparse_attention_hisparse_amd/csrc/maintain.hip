// maintain.hip -- keeping the tiers consistent around the resolver (gfx950):
//  - the row mirror (eager backup): device rows written by the forward pass
//    are copied back to their host rows ("gogongxt.com HiSparse" page, the
//    per-step flow, step 5; "vLLM Hybrid HiSparse 源码实现分析" section 6,
//    the row mirror that lets a later spill move no data);
//  - hot-entry invalidation: hot slots whose rows were rewritten or whose
//    host rows were reused are emptied (same page, section 6, hot-cache
//    coherence).
#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu4;

// One wavefront per (entry, layer), lane l carrying 16-byte unit l; the
// stores go to device-mapped pinned host memory across the host link.
__global__ __launch_bounds__(kCopyThreads) void mirror_rows_kernel(MirrorParams p) {
  constexpr int kWavesPerBlock = kCopyThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int l = p.layer_begin + blockIdx.y;
  const int U = p.units;
  const int64_t hrows = p.host_rows_of_layer[l];
  int trips = 0;
  for (int e = blockIdx.x * kWavesPerBlock + wv; e < p.count; e += gridDim.x * kWavesPerBlock) {
    const int d = __builtin_amdgcn_readfirstlane(p.dev_rows[e]);
    const int64_t hv = p.host_rows[e];
    const int64_t h = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)hv) |
                      ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(hv >> 32)) << 32);
    if (d < 0) continue;  // padding entry
    if ((int64_t)d >= p.dev_pool_rows || h < 0 || h >= hrows) {
      ++trips;
      continue;
    }
    const gu4* src = (const gu4*)p.dev_pools[l] + (int64_t)d * U;
    gu4* dst = (gu4*)p.host_pools[l] + h * U;
    for (int part = lane; part < U; part += kWave) dst[part] = src[part];
  }
  if (trips && lane == 0 && p.stats) atomicAdd(&p.stats[4], (unsigned long long)trips);
}

// One workgroup per entry: every slot of the request row is compared with
// the token range.
__global__ __launch_bounds__(256) void invalidate_tokens_kernel(InvalidateParams p) {
  const int i = blockIdx.x;
  const int r = p.req_rows[i];
  if (r < 0) return;  // padding
  if (r >= p.R) {
    if (threadIdx.x == 0 && p.stats) atomicAdd(&p.stats[4], 1ull);
    return;
  }
  const int lo = p.tok_begin[i], hi = p.tok_end[i];
  int32_t* st = p.slot_tokens + (int64_t)r * p.S;
  int32_t* lru = p.lru_slots + (int64_t)r * p.S;
  for (int s = threadIdx.x; s < p.S; s += 256) {
    const int t = st[s];
    if (t >= lo && t < hi) {
      st[s] = -1;
      lru[s] = 0;
    }
  }
}

// kInvSlotsPerThread consecutive slots (of the flattened [R][S] state) per
// thread, kInvThreads threads per workgroup; the sorted set is staged in LDS
// once per workgroup.  Each slot's host row is looked up with a branch-free
// lower bound of a fixed step count; a thread's searches advance together.
// Measured on 72 requests x 4096 slots against 4096 rows: 512 x 1 takes
// 9.6 us, 256 x 1 11.5, 1024 x 1 9.8, 512 x 2 11.8, 1024 x 4 15.3.
constexpr int kInvThreads = 512;
constexpr int kInvSlotsPerThread = 1;

__device__ inline int lower_bound_fixed(const int64_t* rows, int count, int64_t h) {
  int base = 0, n = count;
  while (n > 1) {
    const int half = n >> 1;
    base = rows[base + half] < h ? base + half : base;
    n -= half;
  }
  return base + (rows[base] < h ? 1 : 0);
}

__global__ __launch_bounds__(kInvThreads) void invalidate_host_rows_kernel(InvalidateParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int64_t* srows = (int64_t*)smem;
  const bool staged = p.count <= kInvalidateLdsRows;
  if (staged)
    for (int j = threadIdx.x; j < p.count; j += kInvThreads) srows[j] = p.rows[j];
  __syncthreads();
  const int64_t* rows = staged ? srows : p.rows;
  const int64_t total = (int64_t)p.R * p.S;
  const int64_t s0 = ((int64_t)blockIdx.x * kInvThreads + threadIdx.x) * kInvSlotsPerThread;
  int64_t h[kInvSlotsPerThread];
  bool live[kInvSlotsPerThread];
#pragma unroll
  for (int q = 0; q < kInvSlotsPerThread; ++q) {
    const int64_t slot = s0 + q;
    const int64_t sc = slot < total ? slot : total - 1;  // in-range index for every load
    const int t = p.slot_tokens[sc];
    live[q] = slot < total && t >= 0 && (int64_t)t < p.max_seq_len;
    const int r = (int)(sc / p.S);
    h[q] = p.host_cache_locs[(int64_t)r * p.max_seq_len + (live[q] ? t : 0)];
  }
#pragma unroll
  for (int q = 0; q < kInvSlotsPerThread; ++q) {
    if (!live[q]) continue;
    const int idx = lower_bound_fixed(rows, p.count, h[q]);
    if (idx < p.count && rows[idx] == h[q]) {
      p.slot_tokens[s0 + q] = -1;
      p.lru_slots[s0 + q] = 0;
    }
  }
}

}  // namespace

hipError_t launch_mirror_rows(const MirrorParams& p, int layers, hipStream_t stream) {
  if (p.count <= 0 || layers <= 0) return hipSuccess;
  constexpr int kWavesPerBlock = kCopyThreads / kWave;
  int blocks = (p.count + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(mirror_rows_kernel, dim3(blocks, layers), dim3(kCopyThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_invalidate_tokens(const InvalidateParams& p, hipStream_t stream) {
  if (p.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(invalidate_tokens_kernel, dim3(p.count), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_invalidate_host_rows(const InvalidateParams& p, hipStream_t stream) {
  if (p.count <= 0) return hipSuccess;
  const int64_t slots = (int64_t)p.R * p.S;
  const int64_t per_block = (int64_t)kInvThreads * kInvSlotsPerThread;
  const size_t lds = p.count <= kInvalidateLdsRows ? (size_t)p.count * sizeof(int64_t) : 0;
  hipLaunchKernelGGL(invalidate_host_rows_kernel, dim3((unsigned)((slots + per_block - 1) / per_block)),
                     dim3(kInvThreads), lds, stream, p);
  return hipGetLastError();
}

hipError_t prepare_maintain() {
  return hipFuncSetAttribute((const void*)invalidate_host_rows_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(kInvalidateLdsRows * sizeof(int64_t)));
}

}  // namespace hisparse
