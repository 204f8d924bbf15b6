// common.h -- internal helpers shared by the HIP kernels of libhisparse
// (gfx950, 64-wide wavefronts).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hisparse {

constexpr int kWave = 64;

// Launch shapes and LDS limits of the resolver.
constexpr int kResolveThreads = 1024;                 // 16 waves per request row
constexpr int kResolveWaves = kResolveThreads / kWave;
constexpr int kMaxTopK = 4096;
constexpr int kMaxSlots = 16384;
constexpr size_t kLdsBudget = 160 * 1024;             // bytes of LDS per CU (gfx950)
constexpr int kVictimRounds = 4;                      // min-extraction rounds before
                                                      // the full sort fallback

// Copy kernel shape.
constexpr int kCopyThreads = 256;

__host__ __device__ inline int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

__host__ __device__ inline int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// Byte offsets of the resolver's dynamic LDS carve-up for S slots and top-k k.
struct ResolveLds {
  int hash_size;   // open-addressing table size (power of two >= 2k)
  int sort_size;   // power of two >= S (fallback sort)
  size_t off_tok, off_stamp, off_flag, off_etok, off_mentry, off_victim;
  size_t off_region, off_hkey, off_hval, off_ehit, off_sort, off_scratch;
  size_t total;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

__host__ __device__ inline ResolveLds resolve_lds_layout(int S, int k) {
  ResolveLds L;
  L.hash_size = next_pow2(2 * k < 64 ? 64 : 2 * k);
  L.sort_size = next_pow2(S);
  size_t o = 0;
  L.off_tok = o;    o = align16(o + 4 * (size_t)S);
  L.off_stamp = o;  o = align16(o + 4 * (size_t)S);
  L.off_flag = o;   o = align16(o + (size_t)S);
  L.off_etok = o;   o = align16(o + 4 * (size_t)k);
  L.off_mentry = o; o = align16(o + 4 * (size_t)k);
  L.off_victim = o; o = align16(o + 4 * (size_t)k);
  // Region used first by the hash table and per-entry hit slots, later (only
  // if needed) by the fallback sort of victim keys.
  L.off_region = o;
  L.off_hkey = o;
  L.off_hval = align16(L.off_hkey + 4 * (size_t)L.hash_size);
  L.off_ehit = align16(L.off_hval + 4 * (size_t)L.hash_size);
  size_t end_hash = align16(L.off_ehit + 4 * (size_t)k);
  L.off_sort = o;
  size_t end_sort = align16(L.off_sort + 8 * (size_t)L.sort_size);
  o = end_hash > end_sort ? end_hash : end_sort;
  L.off_scratch = o; o = align16(o + 8 * (size_t)kResolveWaves * 2);
  L.total = o;
  return L;
}

}  // namespace hisparse
