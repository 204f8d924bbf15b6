// mla_decode.hip -- sparse-MLA decode attention over resolved rows (gfx950).
//
// For batch row b and head h:  O = softmax(scale * q . K_i) V_i over the rows
// i named by device_buffer_locs, where a 656-byte row holds 512 fp8 (OCP
// e4m3) latent values with one fp32 scale per 128, then 64 bf16 rope values
// ("vLLM Hybrid HiSparse 源码实现分析", section 9); K_i = [latent*scale; rope],
// V_i = latent*scale.  This is the consumer of the resolver's row IDs
// ("vLLM HiSparse 本地 KV 卸载架构": the attention backend reads the device
// cache through physical row IDs).
//
// One workgroup of 4 wavefronts per (batch row, group of 32 heads):
//  - waves 2,3 (producers) load 32 rows per block two blocks ahead into
//    registers, dequantise the latent (fp8 -> f32, times the scale, RNE to
//    bf16) and write a bf16 tile [32 keys][576 (+8 pad) dims] to LDS;
//    double-buffered, one barrier per block;
//  - waves 0,1 (consumers) own 16 heads each: S^T = K Q^T on
//    v_mfma_f32_16x16x32_bf16 with Q in registers, an online softmax, and
//    O^T += V^T P^T where P^T comes straight from the S^T accumulator layout
//    and V^T fragments are read from the same row-major tile with the LDS
//    transpose load (ds_read_b64_tr_b16).
// Workgroups are numbered so that the head groups of one batch row land on
// the same XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

constexpr int kKB = 32;                           // keys per block
constexpr int kLat = 512, kDim = 576;
constexpr int kTileStride = 584;                  // bf16 per tile row (576 + 8 pad)
constexpr int kRowStrideBytes = kTileStride * 2;  // 1168: conflict-free b128 / tr16 reads
constexpr int kTileBytes = kKB * kRowStrideBytes;
constexpr int kHeadsPerWave = 16;
constexpr int kHeadsPerGroup = 32;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const __bf16 x = (__bf16)a, y = (__bf16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// 8 e4m3 bytes (two words) times the block scale -> 8 bf16.
__device__ inline uint4 dequant8(uint32_t w0, uint32_t w1, float sc) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
  return make_uint4(pack_bf16x2(a.x * sc, a.y * sc), pack_bf16x2(b.x * sc, b.y * sc),
                    pack_bf16x2(c.x * sc, c.y * sc), pack_bf16x2(d.x * sc, d.y * sc));
}

// One producer thread's share of one block of one row: the four threads of a
// row take its 16-byte chunks in turn (thread `part` takes latent chunks
// 4e+part, e = 0..7, and rope chunks part and part+4), so at every step the
// four threads touch neighbouring 16-byte chunks -- coalesced loads and
// bank-spread LDS stores.  Chunk 4e+part lies in scale block e/2.
struct RawPart {
  uint4 lat[8];
  uint4 rope[2];
  float4 scale;
  bool valid;
};

// Location of this thread's key in block `blk` (clamped, always in range).
__device__ inline int loc_of(const DecodeParams& p, const int32_t* locb, int blk, int key) {
  const int kk = blk * kKB + key;
  return locb[kk < p.k ? kk : p.k - 1];
}

// Issue the loads of one row share; `loc` was fetched two blocks earlier, so
// no load here waits on another.  Keys past k and invalid locations read
// row 0 and are stored as zeros.
__device__ inline void load_part(RawPart& R, const DecodeParams& p, int blk, int key, int loc,
                                 int part) {
  R.valid = (blk * kKB + key < p.k) && loc >= 0 && (int64_t)loc < p.pool_rows;
  const unsigned char* row = p.pool + (int64_t)(R.valid ? loc : 0) * p.row_bytes;
  const uint4* chunks = (const uint4*)row;
#pragma unroll
  for (int e = 0; e < 8; ++e) R.lat[e] = chunks[4 * e + part];
  R.scale = *(const float4*)(row + kLat);
  const uint4* rope = (const uint4*)(row + kLat + 16);
  R.rope[0] = rope[part];
  R.rope[1] = rope[part + 4];
}

__device__ inline void store_part(const RawPart& R, unsigned char* tile, uint8_t* vflag, int key,
                                  int part) {
  uint4* row = (uint4*)(tile + key * kRowStrideBytes);  // 16-byte units of bf16
  if (R.valid) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float sc = (e >> 1) == 0 ? R.scale.x : (e >> 1) == 1 ? R.scale.y
                     : (e >> 1) == 2 ? R.scale.z : R.scale.w;
      const int c = 4 * e + part;  // 16 fp8 -> 32 bytes of bf16 at unit 2c
      row[2 * c] = dequant8(R.lat[e].x, R.lat[e].y, sc);
      row[2 * c + 1] = dequant8(R.lat[e].z, R.lat[e].w, sc);
    }
    row[kLat / 8 + part] = R.rope[0];
    row[kLat / 8 + part + 4] = R.rope[1];
  } else {  // masked key: zeros, so that 0-weight products stay finite
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      row[2 * (4 * e + part)] = z;
      row[2 * (4 * e + part) + 1] = z;
    }
    row[kLat / 8 + part] = z;
    row[kLat / 8 + part + 4] = z;
  }
  if (part == 0) vflag[key] = R.valid ? 1 : 0;
}

__global__ __launch_bounds__(256, 2) void sparse_mla_decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int HG = (p.heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int x = blockIdx.x;
  const int b = (x / (8 * HG)) * 8 + (x % 8);
  const int hg = (x / 8) % HG;
  if (b >= p.batch) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int nb = (p.k + kKB - 1) / kKB;
  const int32_t* locb = p.locs + (int64_t)b * p.k;
  uint8_t* vflags = smem + 2 * kTileBytes;

  if (nb == 0) {  // no entries: O = 0
    if (wave < 2) {
      const int h = hg * kHeadsPerGroup + wave * kHeadsPerWave + r16;
      if (h < p.heads) {
        uint16_t* orow = p.out + ((int64_t)b * p.heads + h) * kLat;
        for (int t = 0; t < kLat / 16; ++t) *(uint2*)(orow + 16 * t + 4 * g) = make_uint2(0u, 0u);
      }
    }
    return;
  }
  if (wave >= 2) {
    // ---------------- producers ----------------
    const int pt = tid - 128;
    const int key = pt >> 2, part = pt & 3;
    // R0 holds even blocks, R1 odd blocks (static indexing keeps them in
    // registers).  Block x is loaded two iterations before it is stored and
    // its location one more iteration before that.
    RawPart R0, R1;
    const int last = nb - 1;
    int la = loc_of(p, locb, 0, key);
    int lb = loc_of(p, locb, min(1, last), key);
    load_part(R0, p, 0, key, la, part);
    la = loc_of(p, locb, min(2, last), key);
    load_part(R1, p, 1, key, lb, part);
    lb = loc_of(p, locb, min(3, last), key);
    store_part(R0, smem, vflags, key, part);
    load_part(R0, p, 2, key, la, part);
    la = loc_of(p, locb, min(4, last), key);
    __syncthreads();
    for (int blk = 0; blk < nb; blk += 2) {
      // iteration blk (even): store block blk+1 (odd, in R1) into buffer 1
      if (blk + 1 < nb) store_part(R1, smem + kTileBytes, vflags + 32, key, part);
      load_part(R1, p, blk + 3, key, lb, part);
      lb = loc_of(p, locb, min(blk + 5, last), key);
      __syncthreads();
      if (blk + 1 >= nb) break;
      // iteration blk+1 (odd): store block blk+2 (even, in R0) into buffer 0
      if (blk + 2 < nb) store_part(R0, smem, vflags, key, part);
      load_part(R0, p, blk + 4, key, la, part);
      la = loc_of(p, locb, min(blk + 6, last), key);
      __syncthreads();
    }
    return;
  }

  // ---------------- consumers ----------------
  const int h0 = hg * kHeadsPerGroup + wave * kHeadsPerWave;
  const int h = h0 + r16;
  const bool head_ok = h < p.heads;
  bf16x8 qf[kDim / 32];
  {
    const bf16x8* qrow = (const bf16x8*)(p.q + ((int64_t)b * p.heads + (head_ok ? h : 0)) * kDim);
#pragma unroll
    for (int ks = 0; ks < kDim / 32; ++ks) qf[ks] = qrow[ks * 4 + g];
  }
  f32x4 o[kLat / 16];
#pragma unroll
  for (int t = 0; t < kLat / 16; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale * 1.4426950408889634f;  // scale * log2(e)
  __syncthreads();

  for (int blk = 0; blk < nb; ++blk) {
    const unsigned char* tile = smem + (blk & 1) * kTileBytes;
    const uint8_t* vf = vflags + 32 * (blk & 1);
    // S^T = K Q^T for the block's 32 keys (two 16-key tiles, two chains each).
    f32x4 s[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m) s[m][0] = s[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDim / 32; ++ks) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 a = *(const bf16x8*)(tile + (16 * m + r16) * kRowStrideBytes + 2 * (32 * ks + 8 * g));
        s[m][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], s[m][ks & 1], 0, 0, 0);
      }
    }
    // Online softmax over this block for head h (column of S^T).
    float xv[2][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const uint32_t vw = *(const uint32_t*)(vf + 16 * m + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sv = s[m][0][i] + s[m][1][i];
        xv[m][i] = ((vw >> (8 * i)) & 0xFF) ? sv * sl2 : -INFINITY;
        mloc = fmaxf(mloc, xv[m][i]);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    float alpha = 1.f;
    float pv[2][4];
    if (m_new == -INFINITY) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[m][i] = 0.f;
    } else {
      alpha = exp2f(m_run - m_new);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[m][i] = exp2f(xv[m][i] - m_new);
    }
    float psum = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) psum += pv[m][i];
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
      for (int t = 0; t < kLat / 16; ++t) o[t] *= alpha;
    }
    // P^T in the B layout: k-slots 0..3 = keys 4g..4g+3, 4..7 = keys 16+4g..16+4g+3.
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pb[i] = (__bf16)pv[0][i];
      pb[4 + i] = (__bf16)pv[1][i];
    }
    // O^T += V^T P^T: the V^T fragment of dims 16t..16t+15 for the same key
    // order, read transposed from the row-major tile.
    const int tk0 = 4 * g + (r16 >> 2);  // key row this lane addresses
    const int td = 4 * (r16 & 3);        // dim offset inside the 16-dim tile
#pragma unroll
    for (int t = 0; t < kLat / 16; ++t) {
      const unsigned char* a0 = tile + tk0 * kRowStrideBytes + 2 * (16 * t + td);
      const unsigned char* a1 = a0 + 16 * kRowStrideBytes;
      const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a0));
      const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(a1));
      const bf16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[t], 0, 0, 0);
    }
    __syncthreads();
  }

  // Normalise by the softmax denominator and store bf16 O[b][h][d].
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (head_ok) {
    uint16_t* orow = p.out + ((int64_t)b * p.heads + h) * kLat;
#pragma unroll
    for (int t = 0; t < kLat / 16; ++t) {
      uint2 w;
      w.x = pack_bf16x2(o[t][0] * inv, o[t][1] * inv);
      w.y = pack_bf16x2(o[t][2] * inv, o[t][3] * inv);
      *(uint2*)(orow + 16 * t + 4 * g) = w;
    }
  }
}

}  // namespace

size_t decode_lds_bytes() { return 2 * (size_t)kTileBytes + 64; }

hipError_t prepare_sparse_mla_decode() {
  return hipFuncSetAttribute((const void*)sparse_mla_decode_kernel,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds_bytes());
}

hipError_t launch_sparse_mla_decode(const DecodeParams& p, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  const int HG = (p.heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int grid = ((batch + 7) / 8) * 8 * HG;
  hipLaunchKernelGGL(sparse_mla_decode_kernel, dim3(grid), dim3(256), decode_lds_bytes(), stream, p);
  return hipGetLastError();
}

}  // namespace hisparse
