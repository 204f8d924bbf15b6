// gather.hip -- miss copy: rows of pinned host memory into hot device rows.
//
// One wavefront per row: lane l carries 16-byte unit l of the row, so each
// row is read from the device-mapped pinned host pages as one contiguous run
// (zero copy; the loads cross the host link).  Workgroups of four
// wavefronts take every (4*chunks)-th entry of one batch row's miss plan.  On
// MI355X the copy is bound by the host link: 656-byte rows straddle 128-byte
// lines, so about 768 bytes cross the link per row.  A plan entry whose host
// row is out of range zero-fills its destination and counts one tripwire.
// Layers sharing one index replay the same plan (grid.y = layer), as the
// follower layers of "vLLM Hybrid HiSparse 源码实现分析" section 7.4; the copy
// itself plays the part of the gather kernel of section 7.2 of that page.
#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

__global__ __launch_bounds__(kCopyThreads) void gather_copy_kernel(CopyParams p) {
  constexpr int kWavesPerBlock = kCopyThreads / kWave;
  const int b = blockIdx.x / p.chunks;
  const int ch = blockIdx.x - b * p.chunks;
  const int l = p.layer_begin + blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  const int m = p.plan_cnt[b];
  const int U = p.units;
  const uint4* __restrict__ hp = (const uint4*)p.host_pools[l];
  uint4* __restrict__ dp = (uint4*)p.dev_pools[l];
  const int64_t hrows = p.host_rows[l];
  const int64_t* __restrict__ psrc = p.plan_src + (int64_t)b * p.plan_stride;
  const int32_t* __restrict__ pdst = p.plan_dst + (int64_t)b * p.plan_stride;
  const int step = p.chunks * kWavesPerBlock;
  for (int e = ch * kWavesPerBlock + wv; e < m; e += step) {
    const int64_t h = psrc[e];
    const int64_t d = (int64_t)pdst[e] * U;
    const bool ok = h >= 0 && h < hrows;
    for (int part = lane; part < U; part += kWave) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (ok) v = hp[h * U + part];
      dp[d + part] = v;
    }
    if (!ok && lane == 0 && p.stats) atomicAdd(&p.stats[4], 1ull);
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
