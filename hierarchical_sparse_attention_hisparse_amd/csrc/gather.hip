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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu4;  // 16 bytes of global memory

// Narrow form, for a copy that runs beside another kernel: gridDim.x
// workgroups of 1024 threads walk the batch rows (grid stride), each
// wavefront copying kNarrowCopyRowsInFlight rows per iteration, so the copy holds
// few CUs while keeping enough rows in flight for the host link.  Row
// indices are wave-uniform; the bytes and tripwires are those of the wide
// form.
__global__ __launch_bounds__(kNarrowCopyThreads) void gather_copy_narrow_kernel(CopyParams p, int batch) {
  constexpr int W = kNarrowCopyThreads / kWave;
  constexpr int RIF = kNarrowCopyRowsInFlight;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int l = p.layer_begin + blockIdx.y;
  const int U = p.units;
  const gu4* hp = (const gu4*)p.host_pools[l];
  gu4* dp = (gu4*)p.dev_pools[l];
  const int64_t hrows = p.host_rows[l];
  int trips = 0;
  for (int b = blockIdx.x; b < batch; b += gridDim.x) {
    const int m = p.plan_cnt[b];
    const int64_t* psrc = p.plan_src + (int64_t)b * p.plan_stride;
    const int32_t* pdst = p.plan_dst + (int64_t)b * p.plan_stride;
    for (int e0 = wv; e0 < m; e0 += W * RIF) {
      int64_t h[RIF];
      int32_t d[RIF];
      bool real[RIF], ok[RIF];
#pragma unroll
      for (int q = 0; q < RIF; ++q) {
        const int e = e0 + q * W;
        real[q] = e < m;
        const int eq = real[q] ? e : e0;
        const int64_t hv = psrc[eq];
        h[q] = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)hv) |
               ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(hv >> 32)) << 32);
        d[q] = __builtin_amdgcn_readfirstlane(pdst[eq]);
        ok[q] = h[q] >= 0 && h[q] < hrows;
        trips += (real[q] && !ok[q]) ? 1 : 0;
      }
      for (int part = lane; part < U; part += kWave) {
        u32x4 v[RIF];
#pragma unroll
        for (int q = 0; q < RIF; ++q) {
          v[q] = u32x4{0u, 0u, 0u, 0u};
          if (real[q] && ok[q]) v[q] = hp[h[q] * U + part];
        }
#pragma unroll
        for (int q = 0; q < RIF; ++q)
          if (real[q]) dp[(int64_t)d[q] * U + part] = v[q];
      }
    }
  }
  if (trips && lane == 0 && p.stats) atomicAdd(&p.stats[4], (unsigned long long)trips);
}

}  // namespace

hipError_t launch_gather_copy_narrow(const CopyParams& p, int batch, int layers, int groups,
                                     hipStream_t stream) {
  if (batch <= 0 || layers <= 0) return hipSuccess;
  const int g = groups < batch ? groups : batch;
  hipLaunchKernelGGL(gather_copy_narrow_kernel, dim3(g, layers), dim3(kNarrowCopyThreads), 0,
                     stream, p, batch);
  return hipGetLastError();
}

hipError_t launch_gather_copy(const CopyParams& p, int batch, int layers, hipStream_t stream) {
  if (batch <= 0 || layers <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_copy_kernel, dim3(batch * p.chunks, layers), dim3(kCopyThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace hisparse
