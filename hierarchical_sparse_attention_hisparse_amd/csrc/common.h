// common.h -- internal helpers shared by the HIP kernels of libhisparse
// (gfx950, 64-wide wavefronts).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hisparse {

constexpr int kWave = 64;

// Launch shapes and LDS limits of the resolver.
constexpr int kResolveThreads = 1024;  // threads per request row
constexpr int kHashFactor = 8;         // table cells per top-k entry
constexpr int kBucketCells = 4;        // cells per bucket of the table (the probe's read)
constexpr int kResolveWaves = kResolveThreads / kWave;
constexpr int kMaxTopK = 4096;
constexpr int kMaxSlots = 16384;
constexpr size_t kLdsBudget = 160 * 1024;             // bytes of LDS per CU (gfx950)
constexpr int kMaxRankBins = 32;                      // consecutive keys ranked per window
constexpr int kMaxRankWindows = 4;                    // windows before the full-sort fallback

// Copy kernel shape.
constexpr int kCopyThreads = 256;

// Smallest batch whose miss copy runs inside the plan kernel.
constexpr int kFuseMinBatch = 8;
constexpr int kMaxFusedLayers = 8;    // layers whose pointers fit the kernel arguments
constexpr int kCopyRowsInFlight = 3;  // rows per wavefront per iteration of the fused copy (measured: 1, 2, 4 and 8 slower)
// The next layer's copy inside a decode launch (pipelined layer loop): rows
// per wavefront per iteration, and about how many workgroups it adds to the
// decode's (batch rows x chunks of each row's misses).
constexpr int kLayerCopyRowsInFlight = 8;
constexpr int kLayerCopyGroups = 128;
constexpr int kLayerCombineGroups = 128;  // workgroups of the previous layer's combine in the same launch

// Invalidation by host rows: sets up to this many rows are searched in LDS.
constexpr int kInvalidateLdsRows = 8192;

// Decode: at most this many key splits per (batch row, head group).
constexpr int kMaxDecodeSplits = 16;
// Decode split workspace per (batch row, 128-head group, split): bf16 partial
// O [128][512] and fp32 (reference, denominator) [128][2].
constexpr size_t kDecodeUnitBytes = 128 * (512 * sizeof(uint16_t) + 2 * sizeof(float));
// The allocation-free decode keeps its split partials in a static device
// array of this many units (33.8 MB): any batch * ceil(heads / 128) <= 256.
constexpr int kNoAllocDecodeUnits = 256;

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
// The open-addressing table and the per-entry hit slots are dead once the
// slots have probed the table, so the victim ranking's per-key slot bitmaps
// (and their word prefixes) and the fallback victim sort reuse their bytes.
constexpr int kResolveScratchInts = 176;

struct ResolveLds {
  int hash_size;   // cells of the table (power of two >= 2k, >= 64)
  int sort_size;   // power of two >= S (fallback sort)
  int words;       // 64-bit words of one slot bitmap: ceil(S / 64)
  int bins;        // keys ranked per window (<= kMaxRankBins), 0 = sort only
  size_t off_hash, off_hidx, off_hcnt, off_ehit, off_sort, off_bits, off_wpre;
  size_t off_etok, off_mentry, off_mhost, off_victim, off_scratch;
  size_t total;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// Workgroup barrier that orders LDS only: it waits for this wavefront's LDS
// operations, not for its global loads and stores (__syncthreads also drains
// the vector-memory counter, so every barrier after a global store or ahead
// of the first use of a global load would wait for that round trip).  Use it
// only where no thread reads, after the barrier, global memory that another
// thread wrote before it.
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Layout for one table size (cells per top-k entry = factor).
__host__ __device__ inline ResolveLds resolve_lds_layout_f(int S, int k, int factor) {
  ResolveLds L;
  L.hash_size = next_pow2(factor * k < 64 ? 64 : factor * k);
  L.sort_size = next_pow2(S);
  size_t o = 0;
  L.off_hash = o;                                               // int32 positions
  L.off_hidx = align16(L.off_hash + 4 * (size_t)L.hash_size);   // uint16 top-k indices
  L.off_hcnt = align16(L.off_hidx + 2 * (size_t)L.hash_size);   // int32 fill count per bucket
  L.off_ehit = align16(L.off_hcnt + 4 * (size_t)(L.hash_size / kBucketCells));
  const size_t end_hash = align16(L.off_ehit + 4 * (size_t)k);
  L.off_sort = o;
  const size_t end_sort = align16(L.off_sort + 8 * (size_t)L.sort_size);
  o = end_hash > end_sort ? end_hash : end_sort;
  // Ranking bitmaps: the larger dead piece of the region above, either the
  // table or what lies past the per-entry hit slots.  Per word of slots:
  // bins + 1 (a padding column) 64-bit bitmap words and 32-bit prefixes.
  L.words = (S + 63) / 64;
  const size_t per_col = 12 * (size_t)L.words;
  const size_t piece1 = L.off_ehit, piece2 = o - end_hash;
  const size_t piece = piece1 > piece2 ? piece1 : piece2;
  const size_t nb = piece / per_col;  // columns, one of them padding
  L.bins = nb < 2 ? 0 : (nb - 1 > (size_t)kMaxRankBins ? kMaxRankBins : (int)(nb - 1));
  L.off_bits = piece1 >= piece2 ? 0 : end_hash;
  L.off_wpre = L.off_bits + 8 * (size_t)L.words * (L.bins + 1);
  L.off_etok = o;    o = align16(o + 4 * (size_t)k);
  L.off_mentry = o;  o = align16(o + 4 * (size_t)k);
  L.off_mhost = o;   o = align16(o + 4 * (size_t)k);
  L.off_victim = o;  o = align16(o + 4 * (size_t)k);
  L.off_scratch = o; o = align16(o + 4 * (size_t)kResolveScratchInts);
  L.total = o;
  return L;
}

// The sparsest table (kHashFactor cells per entry, down to 2) that fits.
inline ResolveLds resolve_lds_layout(int S, int k) {
  ResolveLds L = resolve_lds_layout_f(S, k, kHashFactor);
  for (int f = kHashFactor / 2; L.total > kLdsBudget && f >= 2; f /= 2) L = resolve_lds_layout_f(S, k, f);
  return L;
}

// Items per thread of the resolver (powers of two).
inline int resolve_slots_per_thread(int S) {
  const int v = (S + kResolveThreads - 1) / kResolveThreads;
  return next_pow2(v < 1 ? 1 : v);
}
inline int resolve_entries_per_thread(int k) {
  const int v = (k + kResolveThreads - 1) / kResolveThreads;
  return next_pow2(v < 1 ? 1 : v);
}
constexpr int kMaxSlotsPerThread = 16;
constexpr int kMaxEntriesPerThread = kMaxTopK / kResolveThreads;  // 4

// Phase trace of the plan kernel (diagnostic build only, HISPARSE_PHASE_TRACE):
// batch rows traced and points per wavefront (8 phase points, then one of
// ranking information).
constexpr int kTraceRows = 256;
constexpr int kTracePoints = 9;

}  // namespace hisparse
