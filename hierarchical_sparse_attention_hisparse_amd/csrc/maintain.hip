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

// One thread per slot of every request row: the slot's host row is looked
// up in the sorted set (staged in LDS when it fits) by binary search.
__global__ __launch_bounds__(256) void invalidate_host_rows_kernel(InvalidateParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  int64_t* srows = (int64_t*)smem;
  const bool staged = p.count <= kInvalidateLdsRows;
  if (staged)
    for (int j = threadIdx.x; j < p.count; j += 256) srows[j] = p.rows[j];
  __syncthreads();
  const int64_t slot = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (slot >= (int64_t)p.R * p.S) return;
  const int r = (int)(slot / p.S);
  const int t = p.slot_tokens[slot];
  if (t < 0 || (int64_t)t >= p.max_seq_len) return;
  const int64_t h = p.host_cache_locs[(int64_t)r * p.max_seq_len + t];
  const int64_t* rows = staged ? srows : p.rows;
  int lo = 0, hi = p.count;  // first index with rows[idx] >= h
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rows[mid] < h) lo = mid + 1;
    else hi = mid;
  }
  if (lo < p.count && rows[lo] == h) {
    p.slot_tokens[slot] = -1;
    p.lru_slots[slot] = 0;
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
  const size_t lds = p.count <= kInvalidateLdsRows ? (size_t)p.count * sizeof(int64_t) : 0;
  hipLaunchKernelGGL(invalidate_host_rows_kernel, dim3((unsigned)((slots + 255) / 256)), dim3(256),
                     lds, stream, p);
  return hipGetLastError();
}

hipError_t prepare_maintain() {
  return hipFuncSetAttribute((const void*)invalidate_host_rows_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(kInvalidateLdsRows * sizeof(int64_t)));
}

}  // namespace hisparse
