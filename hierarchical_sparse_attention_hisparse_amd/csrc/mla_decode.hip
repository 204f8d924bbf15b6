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
// One workgroup of 4 wavefronts per (batch row, group of 128 heads, split of
// the keys).  All four wavefronts share the loading: each block of 32 keys is
// fetched a block ahead into registers, then dequantised (fp8 -> f32, times
// the scale, RNE to bf16) and written to one of three bf16 tiles
// [32 keys][576 (+8 pad) dims] in LDS between the MFMAs of the previous
// block's score loop.  With three tiles and two P buffers, the one barrier
// per block (after P is published) also orders every tile reuse.  Each wavefront
// computes the scores of its own 32 heads, so every K fragment read from LDS
// feeds two MFMAs (instruction issue, not bytes, bounds this loop on gfx950),
// and then O for a quarter of the dims of all 128 heads, so every
// transposed V fragment is read once per workgroup and feeds eight MFMAs:
//  - S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with Q held in registers;
//  - a softmax against a fixed reference per head: the maximum of the first
//    block holding a valid key for that head.  P = 2^(x - ref) is exact in
//    fp32 and bf16 for any x up to ref + 64 (log2 units), so O is never
//    rescaled in the loop (a conditional rescale of the accumulator registers
//    forces the compiler to spill them).  If some score exceeds its reference
//    by more than that, the workgroup runs a second pass over its keys with a
//    reference that the first pass has shown to be high enough;
//  - P^T fragments taken straight from the S^T accumulator layout (keys
//    permuted consistently) are exchanged through LDS (the block's one
//    barrier);
//  - O^T += V^T P^T with the V^T fragments read from the same row-major tile
//    with the LDS transpose load (ds_read_b64_tr_b16).
// Each workgroup writes its O normalised by its own denominator (bf16) with
// its reference and denominator (fp32); a second kernel combines the splits
// (the same algebra as one pass, in fp32).
//
// For the layer pipeline (copy of layer l+1 under the attention of layer l,
// "vLLM Hybrid HiSparse 源码实现分析" section 6), a second instance of the
// kernel takes extra workgroups after the decode's: first some that copy the
// next layer's misses from pinned host memory, then some that combine the
// previous layer's splits with the combine kernel's own function.  They run
// on the CUs the decode leaves free and on those its workgroups release, in
// the same launch, so the pipeline needs no second stream.
#include "common.h"
#include "kernels.h"

namespace hisparse {

namespace {

constexpr int kKB = 32;                           // keys per block
constexpr int kLat = 512, kDim = 576;
// bf16 per tile row (576 + 8 pad).  The bank-conflict counter shows 2-way
// conflicts at this 1168-byte stride on the b128 K reads and the tr16 V reads
// (1184 bytes is conflict-free on both), but the kernel measures no faster
// at 1184: LDS is not what bounds it.
constexpr int kTileStride = 584;
constexpr int kRowStrideBytes = kTileStride * 2;
constexpr int kTileBytes = kKB * kRowStrideBytes;
constexpr int kDecWaves = 4;
constexpr int kHeadsPerWave = 32;
constexpr int kHeadsPerGroup = kDecWaves * kHeadsPerWave;  // 128
constexpr float kMaxExcessLog2 = 64.f;            // largest score above a head's reference (log2)
constexpr int kQRopeStrideBytes = 144;            // 64 bf16 + 16 pad: conflict-free b128 reads
constexpr int kLatSteps = kLat / 32;              // 16 k-steps over the latent
constexpr int kQKAhead = 3;                       // LDS reads this many MFMA steps ahead (measured: 1 and 2 slower, 4 no faster)
constexpr int kTiles = 3;                         // K/V tiles in flight (read, PV, written)
constexpr size_t kOffFlags = kTiles * (size_t)kTileBytes;
// per tile: 32 float biases, 0 for a valid key and -inf for a masked one
constexpr size_t kOffOvf = kOffFlags + kTiles * 32 * sizeof(float);  // int: a score exceeded its reference by > 2^64
constexpr size_t kOffQRope = kOffOvf + 16;        // [128 heads][72 bf16] rope part of Q
constexpr int kHeadTiles = kHeadsPerGroup / 16;    // 8
constexpr int kDimTilesPerWave = kLat / 16 / kDecWaves;  // 8: O dims 128w..128w+127
constexpr size_t kOffP = kOffQRope + (size_t)kHeadsPerGroup * kQRopeStrideBytes;  // P^T fragments
constexpr size_t kPBytes = (size_t)kHeadTiles * 64 * 16;
static_assert(kDecodeUnitBytes == kHeadsPerGroup * (kLat * sizeof(uint16_t) + 2 * sizeof(float)),
              "split workspace unit");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16x2(float a, float b) {  // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
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

// One thread's share of one key row: the eight threads of a key take its
// 16-byte latent chunks part, part+8, part+16, part+24 (chunk part+8e lies in
// scale block e) and rope chunk `part`, so neighbouring threads touch
// neighbouring chunks.
struct RawPart {
  uint4 lat[4];
  uint4 rope;
  float4 scale;
  bool valid;
};

// Workgroup barrier for LDS traffic only: the wave's LDS operations complete,
// while its global loads (rows of the blocks ahead) stay in flight across it.
// __syncthreads() would also wait for those loads, one memory latency per
// barrier.  The memory clobber keeps the compiler from moving LDS accesses
// across it.

// Location of top-k entry `kk` of this row, at a clamped (in-range) index.
__device__ inline int loc_at(const DecodeParams& p, const int32_t* locb, int kk) {
  return locb[kk < p.k ? kk : p.k - 1];
}

// Issue the loads of one row share.  Entries past k and invalid locations
// read row 0 and are stored as zeros.
__device__ inline void load_part(RawPart& R, const DecodeParams& p, int kk, int loc, int part) {
  R.valid = kk < p.k && loc >= 0 && (int64_t)loc < p.pool_rows;
  const unsigned char* row = p.pool + (int64_t)(R.valid ? loc : 0) * p.row_bytes;
  const uint4* chunks = (const uint4*)row;
#pragma unroll
  for (int e = 0; e < 4; ++e) R.lat[e] = chunks[part + 8 * e];
  R.scale = *(const float4*)(row + kLat);
  R.rope = ((const uint4*)(row + kLat + 16))[part];
}

// Dequantise half h (8 values) of latent chunk e of this thread's share and
// write it (16 bytes of bf16) to the key's tile row; a masked key writes
// zeros.  Branch-free, so that it can sit between the MFMAs of the score loop.
__device__ inline void store_half(const RawPart& R, unsigned char* tile, int key, int part, int e,
                                  int h) {
  uint4* row = (uint4*)(tile + key * kRowStrideBytes);  // 16-byte units of bf16
  // A masked key dequantises zero bytes with a zero scale: exact zeros, even
  // where the row it was read from holds NaN codes.
  const float sc = R.valid ? (e == 0 ? R.scale.x : e == 1 ? R.scale.y : e == 2 ? R.scale.z : R.scale.w)
                           : 0.f;
  const uint32_t m = R.valid ? ~0u : 0u;
  const uint4 v = h == 0 ? dequant8(R.lat[e].x & m, R.lat[e].y & m, sc)
                         : dequant8(R.lat[e].z & m, R.lat[e].w & m, sc);
  row[2 * (part + 8 * e) + h] = v;  // 16 fp8 -> 32 bytes of bf16 at unit 2c, c = part + 8e
}

__device__ inline void store_chunk(const RawPart& R, unsigned char* tile, int key, int part, int e) {
  store_half(R, tile, key, part, e, 0);
  store_half(R, tile, key, part, e, 1);
}

// The rope chunk and the key's validity flag.
__device__ inline void store_tail(const RawPart& R, unsigned char* tile, float* vbias, int key,
                                  int part) {
  uint4* row = (uint4*)(tile + key * kRowStrideBytes);
  const uint32_t m = R.valid ? ~0u : 0u;
  row[kLat / 8 + part] = make_uint4(R.rope.x & m, R.rope.y & m, R.rope.z & m, R.rope.w & m);
  if (part == 0) vbias[key] = R.valid ? 0.f : -INFINITY;
}

__device__ inline void store_part(const RawPart& R, unsigned char* tile, float* vbias, int key,
                                  int part) {
#pragma unroll
  for (int e = 0; e < 4; ++e) store_chunk(R, tile, key, part, e);
  store_tail(R, tile, vbias, key, part);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu4;  // 16 bytes of global memory

// The copy role of workgroup g of the batch * copy_chunks launched past the
// decode's own: chunk c of batch row b (g = b * copy_chunks + c) takes every
// (4 * copy_chunks)-th miss of that row, from the copied layer's host pool
// into its device pool, one wavefront per 656-byte row (lane l carries
// 16-byte unit l) and kLayerCopyRowsInFlight rows in flight per wavefront.
// The first of these workgroups run on the CUs the decode leaves free, the
// rest as decode workgroups finish.  A host row outside the pool writes zeros
// and counts a tripwire, as in the separate copy kernel.
__device__ inline void layer_copy(const DecodeParams& p, int g) {
  constexpr int RIF = kLayerCopyRowsInFlight;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int U = p.units;
  const gu4* hp = (const gu4*)p.copy_host;
  gu4* dp = (gu4*)p.copy_dev;
  const int b = g / p.copy_chunks, c = g - b * p.copy_chunks;
  const int stride = kDecWaves * p.copy_chunks;
  int trips = 0;
  {
    const int m = p.plan_cnt[b];
    const int64_t* psrc = p.plan_src + (int64_t)b * p.plan_stride;
    const int32_t* pdst = p.plan_dst + (int64_t)b * p.plan_stride;
    for (int e0 = c * kDecWaves + wv; e0 < m; e0 += stride * RIF) {
      int64_t h[RIF];
      int32_t d[RIF];
      bool real[RIF], ok[RIF];
#pragma unroll
      for (int q = 0; q < RIF; ++q) {
        const int e = e0 + q * stride;
        real[q] = e < m;
        const int eq = real[q] ? e : e0;
        const int64_t hv = psrc[eq];
        h[q] = (int64_t)__builtin_amdgcn_readfirstlane((uint32_t)hv) |
               ((int64_t)__builtin_amdgcn_readfirstlane((uint32_t)(hv >> 32)) << 32);
        d[q] = __builtin_amdgcn_readfirstlane(pdst[eq]);
        ok[q] = h[q] >= 0 && h[q] < p.copy_host_rows;
        trips += (real[q] && !ok[q]) ? 1 : 0;
      }
      for (int part = lane; part < U; part += 64) {
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

// Combine the splits of every (batch row, head): O = sum_j w_j l_j O_j /
// sum_j w_j l_j with w_j = 2^(m_j - max m), O_j the normalised partials.
// One thread per 8 output dims: thread tid of block bx of batch row b, so
// every index is 32-bit shifts and masks.  All splits' (m, l) pairs and
// partial rows (at most NSMAX) are loaded before any is combined.
template <int NSMAX>
__device__ inline void combine_rows(const uint16_t* part_o, const float* part_ml, uint16_t* out,
                                    int heads, int splits, int bx, int b, int tid) {
  const int t = bx * 256 + tid;  // over heads x (kLat / 8)
  const int h = t / (kLat / 8), q = t % (kLat / 8);
  if (h >= heads) return;
  const int HG = (heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int hg = h / kHeadsPerGroup, hl = h % kHeadsPerGroup;
  const int NS = splits;
  const int64_t e0 = ((int64_t)(b * HG + hg) * NS) * kHeadsPerGroup + hl;
  f32x2 ml[NSMAX];
  uint4 v[NSMAX];
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < NSMAX; ++j) {
    ml[j] = f32x2{-INFINITY, 0.f};
    v[j] = make_uint4(0u, 0u, 0u, 0u);
    if (j < NS) {
      const int64_t e = e0 + (int64_t)j * kHeadsPerGroup;
      ml[j] = *(const f32x2*)(part_ml + 2 * e);
      v[j] = *(const uint4*)(part_o + e * kLat + 8 * q);
    }
    M = fmaxf(M, ml[j].x);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  // A NaN score (a NaN code or scale in an attended row) leaves its split's
  // denominator NaN; the softmax it belongs to is NaN, so is the output.
  bool nan_l = false;
#pragma unroll
  for (int j = 0; j < NSMAX; ++j) nan_l |= j < NS && ml[j].y != ml[j].y;
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < NSMAX; ++j) {
      if (j < NS && ml[j].x != -INFINITY) {
        const float wl = exp2f(ml[j].x - M) * ml[j].y;
        L += wl;
        const uint32_t wd[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          acc[2 * k] += wl * __uint_as_float(wd[k] << 16);
          acc[2 * k + 1] += wl * __uint_as_float(wd[k] & 0xFFFF0000u);
        }
      }
    }
  }
  const float inv = nan_l ? __builtin_nanf("") : L > 0.f ? 1.f / L : 0.f;
  uint4 w;
  w.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  w.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  w.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *(uint4*)(out + ((int64_t)b * heads + h) * kLat + 8 * q) = w;
}

// The combine role of workgroup g of the comb_groups launched after the
// copy's: the combine of the previous layer's splits (the same arithmetic
// as the combine kernel), block by block over (batch row, block of 256
// threads).
__device__ inline void combine_role(const DecodeParams& p, int g) {
  const int xb = (p.heads * (kLat / 8) + 255) / 256;
  const int total = xb * p.batch;
  for (int cb = g; cb < total; cb += p.comb_groups) {
    const int b = cb / xb, bx = cb - b * xb;
    if (p.splits <= 2)
      combine_rows<2>(p.comb_part_o, p.comb_part_ml, p.comb_out, p.heads, p.splits, bx, b, threadIdx.x);
    else if (p.splits <= 4)
      combine_rows<4>(p.comb_part_o, p.comb_part_ml, p.comb_out, p.heads, p.splits, bx, b, threadIdx.x);
    else if (p.splits <= 8)
      combine_rows<8>(p.comb_part_o, p.comb_part_ml, p.comb_out, p.heads, p.splits, bx, b, threadIdx.x);
    else
      combine_rows<16>(p.comb_part_o, p.comb_part_ml, p.comb_out, p.heads, p.splits, bx, b, threadIdx.x);
  }
}

// ROLES: the instance of the layer pipeline, whose workgroups past the
// decode's copy another layer's misses, then combine the previous layer's
// splits (uniform per workgroup, before any barrier).  A separate instance,
// because the extra code costs the plain decode scalar-register spills.
template <bool ROLES>
__global__ __launch_bounds__(256, 1) void sparse_mla_decode_kernel(DecodeParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  if constexpr (ROLES) {
    if ((int)blockIdx.x >= p.decode_blocks) {
      const int x = (int)blockIdx.x - p.decode_blocks, ncopy = p.batch * p.copy_chunks;
      if (x < ncopy)
        layer_copy(p, x);
      else
        combine_role(p, x - ncopy);
      return;
    }
  }
  const int HG = (p.heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int NS = p.splits;
  int x = blockIdx.x;
  const int sp = x % NS;
  x /= NS;
  const int hg = x % HG;
  const int b = x / HG;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int nb = (p.k + kKB - 1) / kKB;
  const int per = (nb + NS - 1) / NS;
  const int blk0 = sp * per;
  const int nblk = max(0, min(nb, blk0 + per) - blk0);
  const int32_t* locb = p.locs + (int64_t)b * p.k;
  float* vbiases = (float*)(smem + kOffFlags);
  // First head of this wave.  Waves past the last head compute on clamped
  // queries and their partials are never read: keeping every wave on the same
  // path keeps the accumulators in registers.
  const int hw = hg * kHeadsPerGroup + wave * kHeadsPerWave;
  const int key = tid >> 3, part = tid & 7;                   // loading role

  // The latent part of Q for this wave's two 16-head tiles in the MFMA B
  // layout (registers); its rope part goes to LDS.
  bf16x8 qf[2][kLatSteps];
  unsigned char* qrope = smem + kOffQRope;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int h = hw + 16 * ht + r16;
    const bf16x8* qrow = (const bf16x8*)(p.q + ((int64_t)b * p.heads + (h < p.heads ? h : 0)) * kDim);
#pragma unroll
    for (int ks = 0; ks < kLatSteps; ++ks) qf[ht][ks] = qrow[ks * 4 + g];
  }
  {  // rope part of Q: 128 heads x 8 chunks of 16 bytes, 4 per thread
    const int HGh = hg * kHeadsPerGroup;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = tid + 256 * j;       // chunk id
      const int hl = c >> 3, ch = c & 7;  // local head, 16-byte chunk of its rope
      const int h = HGh + hl;
      const uint4* src = (const uint4*)(p.q + ((int64_t)b * p.heads + (h < p.heads ? h : 0)) * kDim + kLat);
      *(uint4*)(qrope + hl * kQRopeStrideBytes + 16 * ch) = src[ch];
    }
  }
  // O^T accumulators of dims 128*wave..+127 (8 tiles of 16) for all 128 heads
  // of the group (8 tiles of 16).
  f32x4 o[kHeadTiles][kDimTilesPerWave];
  float m_run[2], l_run[2];
  float m_ref2[2] = {-INFINITY, -INFINITY};
  const float sl2 = p.scale * 1.4426950408889634f;  // scale * log2(e)
  int* s_ovf = (int*)(smem + kOffOvf);

#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int ht = 0; ht < kHeadTiles; ++ht)
#pragma unroll
      for (int t = 0; t < kDimTilesPerWave; ++t) o[ht][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      m_run[ht] = m_ref2[ht];  // -inf in the first pass: set by the first valid block
      l_run[ht] = 0.f;
    }
    float m_hi[2] = {-INFINITY, -INFINITY};
    int ovf = 0;
    if (tid == 0) *s_ovf = 0;

    RawPart R;
    int loc_n = 0;
    if (nblk > 0) {
      const int last = nb - 1;
      load_part(R, p, blk0 * kKB + key, loc_at(p, locb, blk0 * kKB + key), part);
      const int loc1 = loc_at(p, locb, min(blk0 + 1, last) * kKB + key);
      loc_n = loc_at(p, locb, min(blk0 + 2, last) * kKB + key);
      store_part(R, smem, vbiases, key, part);
      load_part(R, p, (blk0 + 1) * kKB + key, loc1, part);
    }
    __syncthreads();

    int tcur = 0;  // tile of block i: i mod kTiles
    for (int i = 0; i < nblk; ++i) {
      const int tnext = tcur == kTiles - 1 ? 0 : tcur + 1;
      const unsigned char* tile = smem + tcur * kTileBytes;
      const float* vb = vbiases + 32 * tcur;
      // Block i+1 goes into the third buffer, last read by block i-2's PV,
      // which every wave finished before the previous barrier (past the end
      // of the split it is written and never read).
      unsigned char* ntile = smem + tnext * kTileBytes;
      float* nvb = vbiases + 32 * tnext;
      bf16x8 pb[2];
      {
        // S^T = K Q^T: 2 key tiles x 2 head tiles, K fragments shared by both head tiles.
        f32x4 s[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) s[kt][0] = s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        // K fragments (and, for the rope steps, Q fragments) are read
        // kQKAhead steps ahead of the MFMAs that use them.
        const unsigned char* ka = tile + r16 * kRowStrideBytes + 16 * g;
        const unsigned char* qa = qrope + (wave * kHeadsPerWave + r16) * kQRopeStrideBytes + 16 * g;
        bf16x8 fa0[kQKAhead + 1], fa1[kQKAhead + 1], fb0[kQKAhead + 1], fb1[kQKAhead + 1];
#pragma unroll
        for (int ks = 0; ks < kDim / 32 + kQKAhead; ++ks) {
          if (ks < kDim / 32) {  // issue the reads of step ks
            const int sl = ks % (kQKAhead + 1);
            fa0[sl] = *(const bf16x8*)(ka + 64 * ks);
            fa1[sl] = *(const bf16x8*)(ka + 16 * kRowStrideBytes + 64 * ks);
            if (ks >= kLatSteps) {
              fb0[sl] = *(const bf16x8*)(qa + 64 * (ks - kLatSteps));
              fb1[sl] = *(const bf16x8*)(qa + 16 * kQRopeStrideBytes + 64 * (ks - kLatSteps));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          const int c = ks - kQKAhead;  // step whose MFMAs issue now
          if (c >= 0) {
            const int sl = c % (kQKAhead + 1);
            const bf16x8 b0 = c < kLatSteps ? qf[0][c < kLatSteps ? c : 0] : fb0[sl];
            const bf16x8 b1 = c < kLatSteps ? qf[1][c < kLatSteps ? c : 0] : fb1[sl];
            s[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0[sl], b0, s[0][0], 0, 0, 0);
            s[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa0[sl], b1, s[0][1], 0, 0, 0);
            s[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1[sl], b0, s[1][0], 0, 0, 0);
            s[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa1[sl], b1, s[1][1], 0, 0, 0);
            // The next block's tile, half a chunk every second step, its VALU
            // work issued between these MFMAs (which run on the matrix core).
            if (c % 2 == 1 && c / 2 < 8) {
              store_half(R, ntile, key, part, c / 4, (c / 2) & 1);
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // then VALU
              }
            }
            if (c == 16) store_tail(R, ntile, nvb, key, part);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        // The loads of block i+2 (always in range), now that R is stored.
        load_part(R, p, (blk0 + i + 2) * kKB + key, loc_n, part);
        loc_n = loc_at(p, locb, min(blk0 + i + 3, nb - 1) * kKB + key);
        // Softmax for head hw+16ht+r16 over the lane's 8 keys (4g..4g+3 and
        // 16+4g..16+4g+3), against the head's reference m_run.
        const f32x4 vbk[2] = {*(const f32x4*)(vb + 4 * g), *(const f32x4*)(vb + 16 + 4 * g)};
        float xv[2][2][4];
        float lmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // raw scores (masked keys -inf); the scale (> 0) is applied below
              xv[ht][kt][e] = s[kt][ht][e] + vbk[kt][e];
              lmax[ht] = fmaxf(lmax[ht], xv[ht][kt][e]);
            }
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) lmax[ht] *= sl2;
        const bool up0 = lmax[0] > m_run[0] + kMaxExcessLog2;
        const bool up1 = lmax[1] > m_run[1] + kMaxExcessLog2;
        if (__ballot(up0 || up1)) {  // first valid block of a head, or an overflow
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) {
            float bm = lmax[ht];
            bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            int nd = (ht == 0 ? up0 : up1) ? 1 : 0;
            nd |= __shfl_xor(nd, 16, 64);
            nd |= __shfl_xor(nd, 32, 64);
            if (nd) {
              if (m_run[ht] == -INFINITY) {
                m_run[ht] = bm;  // nothing accumulated yet: no rescale needed
              } else {
                ovf = 1;
                m_hi[ht] = fmaxf(m_hi[ht], bm);
              }
            }
          }
        }
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          float pv[2][4];
          float ps = 0.f;
          // no valid key seen yet: every x is -inf, and a finite reference
          // keeps x - ref at -inf (P = 0) instead of NaN
          const float mref = m_run[ht] == -INFINITY ? 0.f : m_run[ht];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // x * sl2 - ref in one fma.  v_exp_f32 without denormal range
              // reduction: results below 2^-126 flush to zero, negligible
              // against the reference's 1.  No clamp: a score more than 64
              // above its reference has set the overflow flag, and the second
              // pass recomputes O and l from zero, so a huge or infinite P of
              // this pass is never used.
              pv[kt][e] = __builtin_amdgcn_exp2f(fmaf(xv[ht][kt][e], sl2, -mref));
              ps += pv[kt][e];
            }
          l_run[ht] += ps;
          // P^T in the B layout: k-slots 0..3 = keys 4g..4g+3, 4..7 = keys 16+4g..16+4g+3.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pb[ht][e] = (__bf16)pv[0][e];
            pb[ht][4 + e] = (__bf16)pv[1][e];
          }
        }
      }
      {
        // Publish this wave's P^T fragments (B layout) for the other waves.
        bf16x8* pbuf = (bf16x8*)(smem + kOffP + (i & 1) * kPBytes);
        pbuf[(2 * wave) * 64 + lane] = pb[0];
        pbuf[(2 * wave + 1) * 64 + lane] = pb[1];
      }
      lds_barrier();  // P of all 128 heads in LDS
      {
        // O^T += V^T P^T over this wave's 128 dims and all 128 heads: every
        // V^T fragment (read transposed from the row-major tile) feeds 8 MFMAs.
        const bf16x8* pbuf = (const bf16x8*)(smem + kOffP + (i & 1) * kPBytes);
        bf16x8 pf[kHeadTiles];
#pragma unroll
        for (int ht = 0; ht < kHeadTiles; ++ht) pf[ht] = pbuf[ht * 64 + lane];
        const int tk0 = 4 * g + (r16 >> 2);  // key row this lane addresses
        const int td = 4 * (r16 & 3);        // dim offset inside the 16-dim tile
        const unsigned char* va0 =
            tile + tk0 * kRowStrideBytes + 2 * (16 * kDimTilesPerWave * wave + td);
        bf16x4 fv0[2], fv1[2];
        fv0[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0));
        fv1[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + 16 * kRowStrideBytes));
#pragma unroll
        for (int t = 0; t < kDimTilesPerWave; ++t) {
          if (t + 1 < kDimTilesPerWave) {  // the next dim tile's fragment
            fv0[(t + 1) & 1] =
                __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(va0 + 32 * (t + 1)));
            fv1[(t + 1) & 1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)(va0 + 16 * kRowStrideBytes + 32 * (t + 1)));
          }
          const bf16x8 va = {fv0[t & 1][0], fv0[t & 1][1], fv0[t & 1][2], fv0[t & 1][3],
                             fv1[t & 1][0], fv1[t & 1][1], fv1[t & 1][2], fv1[t & 1][3]};
#pragma unroll
          for (int ht = 0; ht < kHeadTiles; ++ht)
            o[ht][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[ht], o[ht][t], 0, 0, 0);
        }
      }
      // No barrier here: the next block writes the third tile and the other
      // P buffer, and this block's are rewritten only after the next block's
      // P barrier, which every wave reaches after this PV.
      tcur = tnext;
    }
    if (ovf) *s_ovf = 1;
    __syncthreads();
    const bool again = *s_ovf != 0;  // workgroup-uniform
    if (!again) break;
    // Second pass: every score is at most max(reference, the largest block
    // maximum that exceeded it), so that bound keeps P within 2^64.
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) m_ref2[ht] = fmaxf(m_run[ht], m_hi[ht]);
    __syncthreads();  // everyone has read the flag before it is cleared
  }

  // Partial result of this split, normalised by its own denominator: bf16
  // O_j / l_j (this wave's 128 dims of every head), and fp32 reference (log2
  // units) and denominator of this wave's 32 heads.  1/l crosses from the
  // head's wave to the dims' waves through LDS.
  const int64_t e0 = ((int64_t)(b * HG + hg) * NS + sp) * kHeadsPerGroup;
  float* s_inv = (float*)smem;  // [128 heads]; the tiles are dead now
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    float l_tot = l_run[ht];
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    const int hl = wave * kHeadsPerWave + 16 * ht + r16;
    if (g == 0) {
      s_inv[hl] = l_tot > 0.f ? 1.f / l_tot : 0.f;
      p.part_ml[2 * (e0 + hl)] = m_run[ht];
      p.part_ml[2 * (e0 + hl) + 1] = l_tot;
    }
  }
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht) {
    const float inv = s_inv[16 * ht + r16];
    uint16_t* po = p.part_o + (e0 + 16 * ht + r16) * kLat + 16 * kDimTilesPerWave * wave + 4 * g;
#pragma unroll
    for (int t = 0; t < kDimTilesPerWave; ++t) {
      uint2 w;
      w.x = pack_bf16x2(o[ht][t][0] * inv, o[ht][t][1] * inv);
      w.y = pack_bf16x2(o[ht][t][2] * inv, o[ht][t][3] * inv);
      *(uint2*)(po + 16 * t) = w;
    }
  }
}


// The combine kernel: grid (blocks of 256 threads per batch row, batch).
template <int NSMAX>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  combine_rows<NSMAX>(p.part_o, p.part_ml, p.out, p.heads, p.splits, blockIdx.x, blockIdx.y, threadIdx.x);
}

}  // namespace

size_t decode_lds_bytes() { return kOffP + 2 * kPBytes; }

int decode_splits(int batch, int heads, int k) {
  const int HG = (heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const int nb = (k + kKB - 1) / kKB;
  int s = 256 / (batch * HG > 0 ? batch * HG : 1);
  if (s > kMaxDecodeSplits) s = kMaxDecodeSplits;
  if (s > nb) s = nb;
  return s < 1 ? 1 : s;
}

size_t decode_workspace_bytes(int batch, int heads, int splits) {
  const int HG = (heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const size_t entries = (size_t)batch * HG * splits * kHeadsPerGroup;
  return entries * (kLat * sizeof(uint16_t) + 2 * sizeof(float));
}

// The largest decode_workspace_bytes of any batch <= max_batch and heads <=
// max_heads: decode_splits keeps batch * groups * splits <= 256 while
// batch * groups <= 256, and takes one split beyond.
size_t decode_workspace_max_bytes(int max_batch, int max_heads) {
  const int HG = (max_heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  const size_t units = (size_t)max_batch * HG > 256 ? (size_t)max_batch * HG : 256;
  return units * kHeadsPerGroup * (kLat * sizeof(uint16_t) + 2 * sizeof(float));
}

hipError_t prepare_sparse_mla_decode() {
  hipError_t e = hipFuncSetAttribute((const void*)sparse_mla_decode_kernel<false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds_bytes());
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute((const void*)sparse_mla_decode_kernel<true>,
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)decode_lds_bytes());
}

hipError_t launch_sparse_mla_decode(const DecodeParams& dp, int batch, hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  DecodeParams p = dp;
  const int HG = (p.heads + kHeadsPerGroup - 1) / kHeadsPerGroup;
  p.decode_blocks = batch * HG * p.splits;
  // A copy beside the decode: each of its workgroups holds a whole CU, so
  // the first take the CUs the decode leaves free and the rest follow the
  // decode workgroups as they finish.
  p.copy_chunks = p.copy_dev ? (kLayerCopyGroups + batch - 1) / batch : 0;
  const int cg = batch * p.copy_chunks;
  // The previous layer's combine, after the copy's workgroups.
  p.comb_groups = p.comb_out ? kLayerCombineGroups : 0;
  if (cg + p.comb_groups > 0)
    hipLaunchKernelGGL(sparse_mla_decode_kernel<true>, dim3(p.decode_blocks + cg + p.comb_groups),
                       dim3(256), decode_lds_bytes(), stream, p);
  else
    hipLaunchKernelGGL(sparse_mla_decode_kernel<false>, dim3(p.decode_blocks), dim3(256),
                       decode_lds_bytes(), stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.defer_combine) return e;
  const int per_row = p.heads * (kLat / 8);
  const dim3 cgrid((unsigned)((per_row + 255) / 256), (unsigned)batch);
  static_assert(kMaxDecodeSplits <= 16, "combine instances");
  if (p.splits <= 2)
    hipLaunchKernelGGL(decode_combine_kernel<2>, cgrid, dim3(256), 0, stream, p);
  else if (p.splits <= 4)
    hipLaunchKernelGGL(decode_combine_kernel<4>, cgrid, dim3(256), 0, stream, p);
  else if (p.splits <= 8)
    hipLaunchKernelGGL(decode_combine_kernel<8>, cgrid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_combine_kernel<16>, cgrid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace hisparse
