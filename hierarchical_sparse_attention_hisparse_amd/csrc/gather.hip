// gather.hip -- miss copy: rows of pinned host memory into hot device rows.
//
// Each workgroup takes every `chunks`-th entry of one batch row's miss plan
// and copies those rows 16 bytes per lane, with the lanes of a wavefront
// spread over consecutive 16-byte units of consecutive rows, so each row is
// read from host memory as one contiguous run.  The loads go straight to the
// device-mapped pinned host pages (zero copy); each lane issues several
// independent loads before its stores to keep many host reads in flight.
// A plan entry whose host row is out of range zero-fills its destination
// and counts one tripwire.  Layers sharing one index replay the same plan
// (grid.y = layer), as the follower layers of "vLLM Hybrid HiSparse
// 源码实现分析" section 7.4; the copy itself plays the part of the gather
// kernel described in section 7.2 of that page.
#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

constexpr int kUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void gather_copy_kernel(CopyParams p) {
  const int b = blockIdx.x / p.chunks;
  const int ch = blockIdx.x - b * p.chunks;
  const int l = p.layer_begin + blockIdx.y;
  const int m = p.plan_cnt[b];
  const int mine = m > ch ? (m - ch + p.chunks - 1) / p.chunks : 0;
  const int U = p.units;
  const int total = mine * U;
  const uint4* __restrict__ hp = (const uint4*)p.host_pools[l];
  uint4* __restrict__ dp = (uint4*)p.dev_pools[l];
  const int64_t hrows = p.host_rows[l];
  const int64_t* __restrict__ psrc = p.plan_src + (int64_t)b * p.plan_stride;
  const int32_t* __restrict__ pdst = p.plan_dst + (int64_t)b * p.plan_stride;

  for (int u0 = threadIdx.x; u0 < total; u0 += kCopyThreads * kUnroll) {
    uint4 v[kUnroll];
    int64_t dst[kUnroll];
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
      const int u = u0 + q * kCopyThreads;
      dst[q] = -1;
      v[q] = make_uint4(0u, 0u, 0u, 0u);
      if (u < total) {
        const int e = u / U;
        const int part = u - e * U;
        const int j = ch + e * p.chunks;
        const int64_t h = psrc[j];
        dst[q] = (int64_t)pdst[j] * U + part;
        if (h >= 0 && h < hrows) {
          v[q] = hp[h * U + part];
        } else if (part == 0 && p.stats) {
          atomicAdd(&p.stats[4], 1ull);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q)
      if (dst[q] >= 0) dp[dst[q]] = v[q];
  }
}

}  // namespace

hipError_t launch_gather_copy(const CopyParams& p, int batch, int layers, hipStream_t stream) {
  if (batch <= 0 || layers <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_copy_kernel, dim3(batch * p.chunks, layers), dim3(kCopyThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace hisparse
