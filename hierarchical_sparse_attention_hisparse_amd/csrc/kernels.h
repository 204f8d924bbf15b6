// kernels.h -- internal launch interfaces of libhisparse (not public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace hisparse {

struct ResolveParams {
  int32_t R, S, k, P;
  int64_t max_seq_len, max_pages, resident_pages;
  const int32_t* req_idx;
  const int32_t* topk;
  const int32_t* seq_lens;
  const int64_t* locs;
  const int32_t* bt;  // may be null
  int32_t* st;
  int32_t* lru;
  int32_t* clk;
  int32_t* out;
  unsigned long long* stats;  // may be null
  int64_t* plan_src;
  int32_t* plan_dst;
  int32_t* plan_cnt;
  int32_t plan_stride;
  ResolveLds lds;  // LDS carve-up for (S, k), filled in by launch_resolve
  // Vector loads of each thread's slot-state run (set by launch_resolve):
  // S % slots-per-thread == 0 and the rows aligned for them.
  int32_t vec_state;
  // Fused miss copy (copy_layers > 0): after planning, the workgroup copies
  // its own misses into layers [0, copy_layers) itself.  The per-layer
  // pointers travel in the kernel arguments (constant, scalar-loaded).
  const unsigned char* host_pool[kMaxFusedLayers];  // device-mapped host pointers
  unsigned char* dev_pool[kMaxFusedLayers];
  int64_t host_rows[kMaxFusedLayers];
  const uint4* zero_row;                   // device, `units` zero 16-byte units
  int32_t units;                           // row_bytes / 16
  int32_t copy_layers;                     // 0 = plan only, else <= kMaxFusedLayers
  int32_t P_shift;  // log2(P) when P is a power of two, else -1 (set by launch_resolve)
};

struct CopyParams {
  const unsigned char* const* host_pools;  // device array [L] of device-mapped host pointers
  unsigned char* const* dev_pools;         // device array [L]
  const int64_t* host_rows;                // device array [L]
  const int64_t* plan_src;
  const int32_t* plan_dst;
  const int32_t* plan_cnt;
  unsigned long long* stats;  // may be null
  int32_t plan_stride;
  int32_t units;       // row_bytes / 16
  int32_t chunks;      // workgroups per batch row
  int32_t layer_begin;
};

struct DecodeParams {
  const unsigned char* pool;  // one layer's device pool
  int64_t pool_rows;
  int32_t row_bytes;
  int32_t heads;
  int32_t k;
  int32_t batch;
  float scale;
  const uint16_t* q;     // bf16 bits [batch][heads][576]
  const int32_t* locs;   // [batch][k]
  uint16_t* out;         // bf16 bits [batch][heads][512]
  int32_t splits;        // key splits per (batch row, 128-head group)
  uint16_t* part_o;      // bf16 [batch][groups][splits][128][512] O of a split / its denominator
  float* part_ml;        // [batch][groups][splits][128][2] reference (log2), denominator
  // Optional copy of another layer's misses (plan slice 0) by workgroups
  // launched past the decode's own: copy_dev == nullptr for none.
  const unsigned char* copy_host;  // device-mapped host pool of the copied layer
  unsigned char* copy_dev;         // its device pool
  int64_t copy_host_rows;
  const int64_t* plan_src;
  const int32_t* plan_dst;
  const int32_t* plan_cnt;
  unsigned long long* stats;       // copy tripwires go to stats[4]; may be null
  int32_t plan_stride;
  int32_t units;                   // row_bytes / 16
  int32_t decode_blocks;           // set by the launch
  int32_t copy_chunks;             // set by the launch: workgroups per batch row of the copy
  // Optional combine of a previous call's splits (same batch, heads and
  // splits) by workgroups launched after the copy's: comb_out == nullptr for
  // none.  defer_combine: leave this call's own combine to a later launch.
  const uint16_t* comb_part_o;
  const float* comb_part_ml;
  uint16_t* comb_out;
  int32_t comb_groups;             // set by the launch
  int32_t defer_combine;
};

struct MirrorParams {
  const int32_t* dev_rows;           // [count]
  const int64_t* host_rows;          // [count]
  int32_t count;
  int32_t units;                     // row_bytes / 16
  int32_t layer_begin;
  int64_t dev_pool_rows;
  const unsigned char* const* dev_pools;  // device array [L]
  unsigned char* const* host_pools;       // device array [L] of device-mapped host pointers
  const int64_t* host_rows_of_layer;      // device array [L]
  unsigned long long* stats;              // may be null
};

struct InvalidateParams {
  int32_t R, S;
  int64_t max_seq_len;
  int32_t count;
  const int32_t* req_rows;   // token ranges: [count]
  const int32_t* tok_begin;
  const int32_t* tok_end;
  const int64_t* rows;       // host rows: [count], sorted ascending
  const int64_t* host_cache_locs;
  int32_t* slot_tokens;
  int32_t* lru_slots;
  unsigned long long* stats;  // may be null
};

hipError_t prepare_resolve(size_t lds_bytes);
hipError_t launch_resolve(ResolveParams p, int batch, hipStream_t stream);
hipError_t launch_gather_copy(const CopyParams& p, int batch, int layers, hipStream_t stream);
hipError_t launch_sparse_mla_decode(const DecodeParams& p, int batch, hipStream_t stream);
hipError_t prepare_sparse_mla_decode();
size_t decode_lds_bytes();
hipError_t launch_mirror_rows(const MirrorParams& p, int layers, hipStream_t stream);
hipError_t launch_invalidate_tokens(const InvalidateParams& p, hipStream_t stream);
hipError_t launch_invalidate_host_rows(const InvalidateParams& p, hipStream_t stream);
hipError_t prepare_maintain();
int decode_splits(int batch, int heads, int k);
size_t decode_workspace_bytes(int batch, int heads, int splits);
size_t decode_workspace_max_bytes(int max_batch, int max_heads);

// Records the message of a failing call for hisparse_last_error (the error
// channel every entry point shares) and returns `code`.
int report_error(int code, const char* fmt, ...);

#ifdef HISPARSE_PHASE_TRACE
// The plan kernel's phase trace (diagnostic build): zeroed, or copied out as
// [kTraceRows][kResolveWaves][kTracePoints][2] uint64; both wait for the device.
hipError_t phase_trace_clear();
hipError_t phase_trace_read(uint64_t* host, size_t count);
#endif

}  // namespace hisparse
