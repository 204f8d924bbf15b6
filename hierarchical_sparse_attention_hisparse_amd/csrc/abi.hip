// abi.hip -- the extern "C" entry points of libhisparse (see include/hisparse.h):
// host-side validation, the pool object and its device workspace, and the
// kernel launches.  No entry point that takes a stream synchronises or reads
// device memory back.
#include <hip/hip_runtime.h>
#include <inttypes.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/hisparse.h"
#include "common.h"
#include "kernels.h"

using namespace hisparse;

struct hisparse_pool {
  hisparse_pool_config cfg;
  int device;
  int64_t device_pool_rows;
  int64_t max_pages;
  // device workspace
  int64_t* plan_src;   // [max_batch][max_top_k]
  int32_t* plan_dst;   // [max_batch][max_top_k]
  int32_t* plan_cnt;   // [max_batch]
  unsigned char** d_host_ptrs;  // [L] device-mapped host pool pointers
  unsigned char** d_dev_ptrs;   // [L]
  int64_t* d_host_rows;         // [L]
  uint4* zero_row;              // row_bytes of zeros (source of out-of-range host rows)
  void* dec_ws;                 // decode split partials (two halves), sized at init
  size_t dec_ws_bytes;
  int32_t* plan_batch;          // host: batch of the last plan of each slice (-1: none)
  // host copies
  unsigned char** dev_ptrs;     // [L]
  unsigned char** host_ptrs;    // [L] device-mapped host pool pointers
  int64_t* host_rows;           // [L]
};

namespace {

thread_local char g_err[1024];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return HISPARSE_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_fail(hipError_t e, const char* what) {
  return fail(HISPARSE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int check_device(const hisparse_pool* pool) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != pool->device)
    return fail(HISPARSE_EINVAL, "current device %d is not the pool's device %d", dev,
                pool->device);
  return HISPARSE_OK;
}

int check_resolve_args(const hisparse_pool* pool, int32_t batch, int32_t top_k,
                       const int32_t* req_idx, const int32_t* top_k_tokens,
                       const int32_t* seq_lens, const int64_t* host_cache_locs,
                       const int32_t* bt, int32_t* slot_tokens, int32_t* lru_slots,
                       int32_t* lru_clock, int32_t* out, uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (batch < 0 || batch > pool->cfg.max_batch)
    return fail(HISPARSE_EINVAL, "batch %d outside [0, max_batch=%d]", batch, pool->cfg.max_batch);
  if (top_k < 0 || top_k > pool->cfg.max_top_k)
    return fail(HISPARSE_EINVAL, "top_k %d outside [0, max_top_k=%d]", top_k, pool->cfg.max_top_k);
  if (batch == 0) return HISPARSE_OK;
  const void* req[] = {req_idx, top_k_tokens, seq_lens, host_cache_locs,
                       slot_tokens, lru_slots, lru_clock, out};
  const char* names[] = {"req_idx", "top_k_tokens", "seq_lens", "host_cache_locs",
                         "slot_tokens", "lru_slots", "lru_clock", "device_buffer_locs"};
  for (int i = 0; i < 8; ++i) {
    const bool topk_array = (i == 1 || i == 7);
    if (req[i] == nullptr && topk_array && top_k == 0) continue;  // empty rows
    if (req[i] == nullptr) return fail(HISPARSE_EINVAL, "%s is NULL", names[i]);
    if (!aligned(req[i], i == 3 ? 8 : 4))
      return fail(HISPARSE_EINVAL, "%s is not aligned to its element size", names[i]);
  }
  if (bt != nullptr) {
    if (pool->cfg.page_size <= 0)
      return fail(HISPARSE_EINVAL, "resident_block_table given but the pool has page_size 0");
    if (!aligned(bt, 4)) return fail(HISPARSE_EINVAL, "resident_block_table is not 4-byte aligned");
  }
  if (stats && !aligned(stats, 8)) return fail(HISPARSE_EINVAL, "stats is not 8-byte aligned");
  return HISPARSE_OK;
}

int launch_plan(hisparse_pool* pool, hipStream_t stream, int32_t batch, int32_t top_k,
                const int32_t* req_idx, const int32_t* top_k_tokens, const int32_t* seq_lens,
                const int64_t* host_cache_locs, const int32_t* bt, int32_t* slot_tokens,
                int32_t* lru_slots, int32_t* lru_clock, int32_t* out, uint64_t* stats,
                int32_t copy_layers, int32_t slice = 0) {
  ResolveParams p;
  p.R = pool->cfg.max_requests;
  p.S = pool->cfg.slots;
  p.k = top_k;
  p.P = pool->cfg.page_size;
  p.max_seq_len = pool->cfg.max_seq_len;
  p.max_pages = pool->max_pages;
  p.resident_pages = pool->cfg.resident_pages;
  p.req_idx = req_idx;
  p.topk = top_k_tokens;
  p.seq_lens = seq_lens;
  p.locs = host_cache_locs;
  p.bt = bt;
  p.st = slot_tokens;
  p.lru = lru_slots;
  p.clk = lru_clock;
  p.out = out;
  p.stats = (unsigned long long*)stats;
  const size_t slice_entries = (size_t)pool->cfg.max_batch * pool->cfg.max_top_k;
  p.plan_src = pool->plan_src + slice * slice_entries;
  p.plan_dst = pool->plan_dst + slice * slice_entries;
  p.plan_cnt = pool->plan_cnt + (size_t)slice * pool->cfg.max_batch;
  p.plan_stride = pool->cfg.max_top_k;
  for (int l = 0; l < kMaxFusedLayers; ++l) {
    const bool have = l < copy_layers;
    p.host_pool[l] = have ? pool->host_ptrs[l] : nullptr;
    p.dev_pool[l] = have ? pool->dev_ptrs[l] : nullptr;
    p.host_rows[l] = have ? pool->host_rows[l] : 0;
  }
  p.zero_row = pool->zero_row;
  p.units = pool->cfg.row_bytes / 16;
  p.copy_layers = copy_layers;
  hipError_t e = launch_resolve(p, batch, stream);
  if (e != hipSuccess) return hip_fail(e, "resolve kernel launch");
  pool->plan_batch[slice] = batch;
  return HISPARSE_OK;
}

// A copy replays plan slice `slice`: its batch must be the plan's, or rows
// of an older, larger plan would be copied over slots that now hold others.
int check_plan_batch(const hisparse_pool* pool, int32_t batch, int32_t slice) {
  const int32_t pb = pool->plan_batch[slice];
  if (pb < 0) return fail(HISPARSE_EINVAL, "no plan has been enqueued into plan slice %d", slice);
  if (batch != pb)
    return fail(HISPARSE_EINVAL, "batch %d differs from the batch %d of the plan in slice %d", batch,
                pb, slice);
  return HISPARSE_OK;
}

// MemAvailable of /proc/meminfo in bytes, or -1 if it cannot be read.
int64_t host_mem_available() {
  FILE* f = fopen("/proc/meminfo", "r");
  if (!f) return -1;
  char line[256];
  int64_t kb = -1;
  while (fgets(line, sizeof line, f)) {
    long long v = 0;
    if (sscanf(line, "MemAvailable: %lld kB", &v) == 1) {
      kb = (int64_t)v;
      break;
    }
  }
  fclose(f);
  return kb < 0 ? -1 : kb * 1024;
}

// Workgroups per batch row of the copy: about 4096 wavefronts in total.
int copy_chunks_for(int batch) {
  int c = 4096 / (4 * (batch > 0 ? batch : 1));
  return c < 4 ? 4 : (c > 64 ? 64 : c);
}

int launch_copy(hisparse_pool* pool, hipStream_t stream, int32_t batch, int32_t lb, int32_t le,
                uint64_t* stats, int32_t slice = 0) {
  CopyParams c;
  c.host_pools = pool->d_host_ptrs;
  c.dev_pools = pool->d_dev_ptrs;
  c.host_rows = pool->d_host_rows;
  const size_t slice_entries = (size_t)pool->cfg.max_batch * pool->cfg.max_top_k;
  c.plan_src = pool->plan_src + slice * slice_entries;
  c.plan_dst = pool->plan_dst + slice * slice_entries;
  c.plan_cnt = pool->plan_cnt + (size_t)slice * pool->cfg.max_batch;
  c.stats = (unsigned long long*)stats;
  c.plan_stride = pool->cfg.max_top_k;
  c.units = pool->cfg.row_bytes / 16;
  c.chunks = copy_chunks_for(batch);
  c.layer_begin = lb;
  hipError_t e = launch_gather_copy(c, batch, le - lb, stream);
  if (e != hipSuccess) return hip_fail(e, "gather copy kernel launch");
  return HISPARSE_OK;
}

}  // namespace

// Split partials of hisparse_sparse_mla_decode_noalloc, for callers that
// cannot allocate: a file-scope device array, one copy per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: its device address comes from
// hipGetSymbolAddress, once per device (noalloc_scratch below), and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[(size_t)kNoAllocDecodeUnits * kDecodeUnitBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once known

// The current device's address of `scratch` (looked up on the device's first
// call, which also sets the decode kernels' LDS limit there).  No allocation.
int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(HISPARSE_EUNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(HISPARSE_EHIP, "hipGetSymbolAddress of the decode scratch on device %d: %s", dev,
                  hipGetErrorString(e));
    }
    if ((e = prepare_sparse_mla_decode()) != hipSuccess) return hip_fail(e, "decode kernel set-up");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HISPARSE_OK;
}

}  // namespace

int hisparse::report_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

extern "C" {

const char* hisparse_last_error(void) { return g_err; }

int hisparse_host_alloc(size_t bytes, void** out) {
  if (!out) return fail(HISPARSE_EINVAL, "out is NULL");
  *out = nullptr;
  if (bytes == 0) return fail(HISPARSE_EINVAL, "bytes is 0");
  const int64_t avail = host_mem_available();
  if (avail >= 0 && (double)bytes > 0.95 * (double)avail)
    return fail(HISPARSE_ENOMEM,
                "%zu bytes of pinned host memory exceed 95%% of the host's MemAvailable "
                "(%" PRId64 " bytes)",
                bytes, avail);
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess || p == nullptr)
    return fail(HISPARSE_ENOMEM, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
  *out = p;
  return ok();
}

int hisparse_host_free(void* ptr) {
  if (!ptr) return ok();
  hipError_t e = hipHostFree(ptr);
  if (e != hipSuccess) return hip_fail(e, "hipHostFree");
  return ok();
}

int hisparse_init_pool(const hisparse_pool_config* cfg, void* const* host_pools,
                       const int64_t* host_pool_rows, void* const* device_pools,
                       int64_t device_pool_rows, hisparse_pool** out) {
  if (!out) return fail(HISPARSE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!cfg) return fail(HISPARSE_EINVAL, "config is NULL");
  const hisparse_pool_config c = *cfg;
  if (c.max_requests <= 0) return fail(HISPARSE_EINVAL, "max_requests must be > 0");
  if (c.slots <= 0 || c.slots > kMaxSlots)
    return fail(HISPARSE_EINVAL, "slots %d outside [1, %d]", c.slots, kMaxSlots);
  if (c.max_top_k <= 0 || c.max_top_k > c.slots || c.max_top_k > kMaxTopK)
    return fail(HISPARSE_EINVAL, "max_top_k %d outside [1, min(slots, %d)]", c.max_top_k, kMaxTopK);
  if (c.max_batch <= 0 || c.max_batch > 65535)
    return fail(HISPARSE_EINVAL, "max_batch %d outside [1, 65535]", c.max_batch);
  if (c.row_bytes <= 0 || c.row_bytes % 16 != 0)
    return fail(HISPARSE_EINVAL, "row_bytes %d is not a positive multiple of 16", c.row_bytes);
  if (c.num_layers <= 0) return fail(HISPARSE_EINVAL, "num_layers must be > 0");
  if (c.page_size < 0 || c.resident_pages < 0 || c.max_steps < 0)
    return fail(HISPARSE_EINVAL, "page_size / resident_pages / max_steps must be >= 0");
  if (c.max_heads < 0 || c.max_heads % 16 != 0 || c.max_heads > 65536)
    return fail(HISPARSE_EINVAL, "max_heads %d must be a multiple of 16 in [0, 65536]", c.max_heads);
  if (c.resident_pages > 0 && c.page_size == 0)
    return fail(HISPARSE_EINVAL, "resident_pages > 0 needs page_size > 0");
  if (c.max_seq_len <= 0 || c.max_seq_len > INT32_MAX)
    return fail(HISPARSE_EINVAL, "max_seq_len must be in [1, 2^31)");
  const int64_t need_rows = (int64_t)c.max_requests * c.slots + c.resident_pages * (int64_t)c.page_size;
  if (device_pool_rows < need_rows || device_pool_rows > INT32_MAX)
    return fail(HISPARSE_EINVAL, "device_pool_rows %lld must be >= R*S + resident_pages*P = %lld and < 2^31",
                (long long)device_pool_rows, (long long)need_rows);
  if (resolve_slots_per_thread(c.slots) > kMaxSlotsPerThread ||
      resolve_entries_per_thread(c.max_top_k) > kMaxEntriesPerThread)
    return fail(HISPARSE_EUNSUPPORTED, "slots %d / max_top_k %d exceed the resolver's per-thread limits",
                c.slots, c.max_top_k);
  const ResolveLds lay = resolve_lds_layout(c.slots, c.max_top_k);
  if (lay.total > kLdsBudget)
    return fail(HISPARSE_EUNSUPPORTED, "slots %d with max_top_k %d need %zu bytes of LDS (> %zu)",
                c.slots, c.max_top_k, lay.total, kLdsBudget);
  if (!host_pools || !host_pool_rows || !device_pools)
    return fail(HISPARSE_EINVAL, "pool arrays are NULL");
  const int L = c.num_layers;
  for (int l = 0; l < L; ++l) {
    if (host_pool_rows[l] < 0 || host_pool_rows[l] > INT32_MAX)
      return fail(HISPARSE_EINVAL, "host_pool_rows[%d] outside [0, 2^31)", l);
    if (host_pool_rows[l] > 0 && (!host_pools[l] || !aligned(host_pools[l], 16)))
      return fail(HISPARSE_EINVAL, "host_pools[%d] is NULL or not 16-byte aligned", l);
    if (!device_pools[l] || !aligned(device_pools[l], 16))
      return fail(HISPARSE_EINVAL, "device_pools[%d] is NULL or not 16-byte aligned", l);
  }

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");

  // Device-side views of the pinned host pools.
  unsigned char** hdev = (unsigned char**)calloc(L, sizeof(void*));
  unsigned char** ddev = (unsigned char**)calloc(L, sizeof(void*));
  if (!hdev || !ddev) {
    free(hdev);
    free(ddev);
    return fail(HISPARSE_ENOMEM, "host allocation failed");
  }
  for (int l = 0; l < L; ++l) {
    ddev[l] = (unsigned char*)device_pools[l];
    if (host_pool_rows[l] == 0) continue;
    void* dp = nullptr;
    e = hipHostGetDevicePointer(&dp, host_pools[l], 0);
    if (e != hipSuccess || dp == nullptr) {
      free(hdev);
      free(ddev);
      (void)hipGetLastError();
      return fail(HISPARSE_EINVAL,
                  "host_pools[%d] is not pinned, device-mapped host memory (use hisparse_host_alloc): %s",
                  l, hipGetErrorString(e));
    }
    hdev[l] = (unsigned char*)dp;
  }

  hisparse_pool* pool = (hisparse_pool*)calloc(1, sizeof(hisparse_pool));
  if (!pool) {
    free(hdev);
    free(ddev);
    return fail(HISPARSE_ENOMEM, "host allocation failed");
  }
  pool->cfg = c;
  pool->device = dev;
  pool->device_pool_rows = device_pool_rows;
  pool->max_pages = c.page_size > 0 ? (c.max_seq_len + c.page_size - 1) / c.page_size : 0;
  pool->dev_ptrs = ddev;
  pool->host_ptrs = hdev;
  pool->host_rows = (int64_t*)malloc((size_t)L * sizeof(int64_t));
  if (!pool->host_rows) {
    free(hdev);
    free(ddev);
    free(pool);
    return fail(HISPARSE_ENOMEM, "host allocation failed");
  }
  memcpy(pool->host_rows, host_pool_rows, (size_t)L * sizeof(int64_t));

  const size_t slices = c.max_steps > 1 ? (size_t)c.max_steps : 1;  // one plan per verification step
  pool->plan_batch = (int32_t*)malloc(slices * sizeof(int32_t));
  if (!pool->plan_batch) {
    free(pool->host_rows);
    free(hdev);
    free(ddev);
    free(pool);
    return fail(HISPARSE_ENOMEM, "host allocation failed");
  }
  for (size_t q = 0; q < slices; ++q) pool->plan_batch[q] = -1;
  const size_t entries = (size_t)c.max_batch * c.max_top_k * slices;
  const size_t bytes_src = entries * 8, bytes_dst = entries * 4;
  const size_t bytes_cnt = (size_t)c.max_batch * slices * 4;
  const size_t bytes_tab = (size_t)L * 8;
  unsigned char* ws = nullptr;
  const size_t total = align16(bytes_src) + align16(bytes_dst) + align16(bytes_cnt) +
                       3 * align16(bytes_tab) + align16((size_t)c.row_bytes);
  e = hipMalloc((void**)&ws, total);
  if (e != hipSuccess) {
    free(pool->plan_batch);
    free(pool->host_rows);
    free(hdev);
    free(ddev);
    free(pool);
    (void)hipGetLastError();
    return fail(HISPARSE_ENOMEM, "hipMalloc(%zu) for the plan workspace: %s", total, hipGetErrorString(e));
  }
  size_t o = 0;
  pool->plan_src = (int64_t*)(ws + o);        o += align16(bytes_src);
  pool->plan_dst = (int32_t*)(ws + o);        o += align16(bytes_dst);
  pool->plan_cnt = (int32_t*)(ws + o);        o += align16(bytes_cnt);
  pool->d_host_ptrs = (unsigned char**)(ws + o); o += align16(bytes_tab);
  pool->d_dev_ptrs = (unsigned char**)(ws + o);  o += align16(bytes_tab);
  pool->d_host_rows = (int64_t*)(ws + o);  o += align16(bytes_tab);
  pool->zero_row = (uint4*)(ws + o);
  e = hipMemset(ws, 0, total);
  if (e == hipSuccess) e = hipMemcpy(pool->d_host_ptrs, hdev, bytes_tab, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(pool->d_dev_ptrs, ddev, bytes_tab, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(pool->d_host_rows, host_pool_rows, bytes_tab, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = prepare_resolve(kLdsBudget);
  if (e == hipSuccess) e = prepare_sparse_mla_decode();
  if (e == hipSuccess) e = prepare_maintain();
  if (e != hipSuccess) {
    (void)hipFree(ws);
    free(pool->plan_batch);
    free(pool->host_rows);
    free(hdev);
    free(ddev);
    free(pool);
    return hip_fail(e, "pool set-up");
  }
  // The decode's split workspace, two halves (the layer pipeline alternates
  // them), sized for every shape the configuration admits.
  if (c.max_heads > 0) {
    const size_t dbytes = 2 * decode_workspace_max_bytes(c.max_batch, c.max_heads);
    e = hipMalloc(&pool->dec_ws, dbytes);
    if (e != hipSuccess || !pool->dec_ws) {
      (void)hipGetLastError();
      (void)hipFree(ws);
      free(pool->plan_batch);
      free(pool->host_rows);
      free(hdev);
      free(ddev);
      free(pool);
      return fail(HISPARSE_ENOMEM, "hipMalloc(%zu) for the decode workspace: %s", dbytes,
                  hipGetErrorString(e));
    }
    pool->dec_ws_bytes = dbytes;
  }
  *out = pool;
  return ok();
}

void hisparse_destroy_pool(hisparse_pool* pool) {
  if (!pool) return;
  if (pool->plan_src) (void)hipFree(pool->plan_src);
  if (pool->dec_ws) (void)hipFree(pool->dec_ws);
  free(pool->dev_ptrs);
  free(pool->host_ptrs);
  free(pool->host_rows);
  free(pool->plan_batch);
  free(pool);
}

int hisparse_resolve_plan(hisparse_pool* pool, void* stream, int32_t batch, int32_t top_k,
                          const int32_t* req_idx, const int32_t* top_k_tokens,
                          const int32_t* seq_lens, const int64_t* host_cache_locs,
                          const int32_t* resident_block_table, int32_t* slot_tokens,
                          int32_t* lru_slots, int32_t* lru_clock, int32_t* device_buffer_locs,
                          uint64_t* stats) {
  int rc = check_resolve_args(pool, batch, top_k, req_idx, top_k_tokens, seq_lens, host_cache_locs,
                              resident_block_table, slot_tokens, lru_slots, lru_clock,
                              device_buffer_locs, stats);
  if (rc != HISPARSE_OK) return rc;
  if (batch == 0) return ok();
  if ((rc = check_device(pool)) != HISPARSE_OK) return rc;
  rc = launch_plan(pool, (hipStream_t)stream, batch, top_k, req_idx, top_k_tokens, seq_lens,
                   host_cache_locs, resident_block_table, slot_tokens, lru_slots, lru_clock,
                   device_buffer_locs, stats, 0);
  return rc == HISPARSE_OK ? ok() : rc;
}

int hisparse_gather_copy(hisparse_pool* pool, void* stream, int32_t batch, int32_t layer_begin,
                         int32_t layer_end, uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (batch < 0 || batch > pool->cfg.max_batch)
    return fail(HISPARSE_EINVAL, "batch %d outside [0, max_batch=%d]", batch, pool->cfg.max_batch);
  if (layer_begin < 0 || layer_end > pool->cfg.num_layers || layer_begin > layer_end)
    return fail(HISPARSE_EINVAL, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end,
                pool->cfg.num_layers);
  if (stats && !aligned(stats, 8)) return fail(HISPARSE_EINVAL, "stats is not 8-byte aligned");
  if (batch == 0 || layer_begin == layer_end) return ok();
  int rc = check_plan_batch(pool, batch, 0);
  if (rc != HISPARSE_OK) return rc;
  if ((rc = check_device(pool)) != HISPARSE_OK) return rc;
  rc = launch_copy(pool, (hipStream_t)stream, batch, layer_begin, layer_end, stats);
  return rc == HISPARSE_OK ? ok() : rc;
}

int hisparse_resolve(hisparse_pool* pool, void* stream, int32_t batch, int32_t top_k,
                     const int32_t* req_idx, const int32_t* top_k_tokens, const int32_t* seq_lens,
                     const int64_t* host_cache_locs, const int32_t* resident_block_table,
                     int32_t* slot_tokens, int32_t* lru_slots, int32_t* lru_clock,
                     int32_t* device_buffer_locs, uint64_t* stats) {
  int rc = check_resolve_args(pool, batch, top_k, req_idx, top_k_tokens, seq_lens, host_cache_locs,
                              resident_block_table, slot_tokens, lru_slots, lru_clock,
                              device_buffer_locs, stats);
  if (rc != HISPARSE_OK) return rc;
  if (batch == 0) return ok();
  if ((rc = check_device(pool)) != HISPARSE_OK) return rc;
  // Large batches copy inside the plan kernel (each request's workgroup
  // copies its own misses, so the copy starts as soon as a plan is ready and
  // there is no second launch); small batches keep the separate copy kernel,
  // whose many wavefronts keep enough rows in flight on the host link.
  const bool fuse = batch >= kFuseMinBatch && pool->cfg.num_layers <= kMaxFusedLayers;
  rc = launch_plan(pool, (hipStream_t)stream, batch, top_k, req_idx, top_k_tokens, seq_lens,
                   host_cache_locs, resident_block_table, slot_tokens, lru_slots, lru_clock,
                   device_buffer_locs, stats, fuse ? pool->cfg.num_layers : 0);
  if (rc != HISPARSE_OK || fuse) return rc == HISPARSE_OK ? ok() : rc;
  rc = launch_copy(pool, (hipStream_t)stream, batch, 0, pool->cfg.num_layers, stats);
  return rc == HISPARSE_OK ? ok() : rc;
}

int hisparse_resolve_steps(hisparse_pool* pool, void* stream, int32_t steps, int32_t batch,
                           int32_t top_k, const int32_t* req_idx, const int32_t* top_k_tokens,
                           const int32_t* seq_lens, const int64_t* host_cache_locs,
                           const int32_t* resident_block_table, int32_t* slot_tokens,
                           int32_t* lru_slots, int32_t* lru_clock, int32_t* device_buffer_locs,
                           uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  const int32_t max_steps = pool->cfg.max_steps > 1 ? pool->cfg.max_steps : 1;
  if (steps < 0 || steps > max_steps)
    return fail(HISPARSE_EINVAL, "steps %d outside [0, max_steps=%d]", steps, max_steps);
  if ((int64_t)steps * top_k > pool->cfg.slots)
    return fail(HISPARSE_EINVAL,
                "steps %d x top_k %d exceed slots %d: a later step could evict a row an earlier "
                "step of the same call still needs",
                steps, top_k, pool->cfg.slots);
  for (int32_t q = 0; q < steps; ++q) {
    const size_t off = (size_t)q * batch * top_k;
    const int32_t* tk = top_k_tokens ? top_k_tokens + off : nullptr;
    int32_t* out = device_buffer_locs ? device_buffer_locs + off : nullptr;
    const int32_t* sl = seq_lens ? seq_lens + (size_t)q * batch : nullptr;
    int rc = check_resolve_args(pool, batch, top_k, req_idx, tk, sl,
                                host_cache_locs, resident_block_table, slot_tokens, lru_slots,
                                lru_clock, out, stats);
    if (rc != HISPARSE_OK) return rc;
    if (batch == 0) return ok();
    if (q == 0 && (rc = check_device(pool)) != HISPARSE_OK) return rc;
    // Each step is planned into its own slice (replayable); steps run in
    // stream order, so step q sees the stamps of steps < q.
    const bool fuse = batch >= kFuseMinBatch && pool->cfg.num_layers <= kMaxFusedLayers;
    rc = launch_plan(pool, (hipStream_t)stream, batch, top_k, req_idx, tk, sl,
                     host_cache_locs, resident_block_table,
                     slot_tokens, lru_slots, lru_clock, out, stats,
                     fuse ? pool->cfg.num_layers : 0, q);
    if (rc != HISPARSE_OK) return rc;
    if (!fuse && (rc = launch_copy(pool, (hipStream_t)stream, batch, 0, pool->cfg.num_layers,
                                   stats, q)) != HISPARSE_OK)
      return rc;
  }
  return ok();
}

int hisparse_gather_copy_step(hisparse_pool* pool, void* stream, int32_t step, int32_t batch,
                              int32_t layer_begin, int32_t layer_end, uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  const int32_t max_steps = pool->cfg.max_steps > 1 ? pool->cfg.max_steps : 1;
  if (step < 0 || step >= max_steps)
    return fail(HISPARSE_EINVAL, "step %d outside [0, max_steps=%d)", step, max_steps);
  if (batch < 0 || batch > pool->cfg.max_batch)
    return fail(HISPARSE_EINVAL, "batch %d outside [0, max_batch=%d]", batch, pool->cfg.max_batch);
  if (layer_begin < 0 || layer_end > pool->cfg.num_layers || layer_begin > layer_end)
    return fail(HISPARSE_EINVAL, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end,
                pool->cfg.num_layers);
  if (stats && !aligned(stats, 8)) return fail(HISPARSE_EINVAL, "stats is not 8-byte aligned");
  if (batch == 0 || layer_begin == layer_end) return ok();
  int rc = check_plan_batch(pool, batch, step);
  if (rc != HISPARSE_OK) return rc;
  if ((rc = check_device(pool)) != HISPARSE_OK) return rc;
  rc = launch_copy(pool, (hipStream_t)stream, batch, layer_begin, layer_end, stats, step);
  return rc == HISPARSE_OK ? ok() : rc;
}

int hisparse_mirror_rows(hisparse_pool* pool, void* stream, int32_t count, const int32_t* dev_rows,
                         const int64_t* host_rows, int32_t layer_begin, int32_t layer_end,
                         uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (count < 0) return fail(HISPARSE_EINVAL, "count %d < 0", count);
  if (layer_begin < 0 || layer_end > pool->cfg.num_layers || layer_begin > layer_end)
    return fail(HISPARSE_EINVAL, "layer range [%d, %d) outside [0, %d)", layer_begin, layer_end,
                pool->cfg.num_layers);
  if (count == 0 || layer_begin == layer_end) return ok();
  if (!dev_rows || !host_rows) return fail(HISPARSE_EINVAL, "dev_rows and host_rows must not be NULL");
  if (!aligned(dev_rows, 4) || !aligned(host_rows, 8))
    return fail(HISPARSE_EINVAL, "dev_rows / host_rows are not aligned to their element size");
  if (stats && !aligned(stats, 8)) return fail(HISPARSE_EINVAL, "stats is not 8-byte aligned");
  int rc = check_device(pool);
  if (rc != HISPARSE_OK) return rc;
  MirrorParams m;
  m.dev_rows = dev_rows;
  m.host_rows = host_rows;
  m.count = count;
  m.units = pool->cfg.row_bytes / 16;
  m.layer_begin = layer_begin;
  m.dev_pool_rows = pool->device_pool_rows;
  m.dev_pools = pool->d_dev_ptrs;
  m.host_pools = pool->d_host_ptrs;
  m.host_rows_of_layer = pool->d_host_rows;
  m.stats = (unsigned long long*)stats;
  hipError_t e = launch_mirror_rows(m, layer_end - layer_begin, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "row mirror kernel launch");
  return ok();
}

int hisparse_invalidate_tokens(hisparse_pool* pool, void* stream, int32_t count,
                               const int32_t* req_rows, const int32_t* tok_begin,
                               const int32_t* tok_end, int32_t* slot_tokens, int32_t* lru_slots,
                               uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (count < 0) return fail(HISPARSE_EINVAL, "count %d < 0", count);
  if (count == 0) return ok();
  if (!req_rows || !tok_begin || !tok_end || !slot_tokens || !lru_slots)
    return fail(HISPARSE_EINVAL, "array arguments must not be NULL");
  if (!aligned(req_rows, 4) || !aligned(tok_begin, 4) || !aligned(tok_end, 4) ||
      !aligned(slot_tokens, 4) || !aligned(lru_slots, 4))
    return fail(HISPARSE_EINVAL, "int32 arrays must be 4-byte aligned");
  if (stats && !aligned(stats, 8)) return fail(HISPARSE_EINVAL, "stats is not 8-byte aligned");
  int rc = check_device(pool);
  if (rc != HISPARSE_OK) return rc;
  InvalidateParams v = {};
  v.R = pool->cfg.max_requests;
  v.S = pool->cfg.slots;
  v.max_seq_len = pool->cfg.max_seq_len;
  v.count = count;
  v.req_rows = req_rows;
  v.tok_begin = tok_begin;
  v.tok_end = tok_end;
  v.slot_tokens = slot_tokens;
  v.lru_slots = lru_slots;
  v.stats = (unsigned long long*)stats;
  hipError_t e = launch_invalidate_tokens(v, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "token invalidation kernel launch");
  return ok();
}

int hisparse_invalidate_host_rows(hisparse_pool* pool, void* stream, int32_t count,
                                  const int64_t* rows_sorted, const int64_t* host_cache_locs,
                                  int32_t* slot_tokens, int32_t* lru_slots) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (count < 0) return fail(HISPARSE_EINVAL, "count %d < 0", count);
  if (count == 0) return ok();
  if (!rows_sorted || !host_cache_locs || !slot_tokens || !lru_slots)
    return fail(HISPARSE_EINVAL, "array arguments must not be NULL");
  if (!aligned(rows_sorted, 8) || !aligned(host_cache_locs, 8) || !aligned(slot_tokens, 4) ||
      !aligned(lru_slots, 4))
    return fail(HISPARSE_EINVAL, "arrays are not aligned to their element size");
  int rc = check_device(pool);
  if (rc != HISPARSE_OK) return rc;
  InvalidateParams v = {};
  v.R = pool->cfg.max_requests;
  v.S = pool->cfg.slots;
  v.max_seq_len = pool->cfg.max_seq_len;
  v.count = count;
  v.rows = rows_sorted;
  v.host_cache_locs = host_cache_locs;
  v.slot_tokens = slot_tokens;
  v.lru_slots = lru_slots;
  hipError_t e = launch_invalidate_host_rows(v, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "host-row invalidation kernel launch");
  return ok();
}

// Argument checks of one decode call (nothing is enqueued).
static int decode_check(hisparse_pool* pool, int32_t batch, int32_t heads, int32_t top_k,
                        int32_t layer, const void* q_bf16, const int32_t* device_buffer_locs,
                        void* out_bf16) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (batch < 0 || batch > pool->cfg.max_batch)
    return fail(HISPARSE_EINVAL, "batch %d outside [0, max_batch=%d]", batch, pool->cfg.max_batch);
  if (heads <= 0 || heads % 16 != 0)
    return fail(HISPARSE_EUNSUPPORTED, "heads %d must be a positive multiple of 16", heads);
  if (heads > pool->cfg.max_heads)
    return fail(HISPARSE_EINVAL, "heads %d exceed the pool's max_heads %d (its decode workspace)",
                heads, pool->cfg.max_heads);
  if (top_k < 0 || top_k > pool->cfg.max_top_k)
    return fail(HISPARSE_EINVAL, "top_k %d outside [0, max_top_k=%d]", top_k, pool->cfg.max_top_k);
  if (layer < 0 || layer >= pool->cfg.num_layers)
    return fail(HISPARSE_EINVAL, "layer %d outside [0, %d)", layer, pool->cfg.num_layers);
  if (pool->cfg.row_bytes < 656)
    return fail(HISPARSE_EUNSUPPORTED, "row_bytes %d is smaller than the 656-byte sparse-MLA row",
                pool->cfg.row_bytes);
  if (batch == 0) return HISPARSE_OK;
  if (!q_bf16 || !out_bf16 || (top_k > 0 && !device_buffer_locs))
    return fail(HISPARSE_EINVAL, "q_bf16, out_bf16 and device_buffer_locs must not be NULL");
  if (!aligned(q_bf16, 16) || !aligned(out_bf16, 8) || !aligned(device_buffer_locs, 4))
    return fail(HISPARSE_EINVAL, "q_bf16 must be 16-byte, out_bf16 8-byte and locs 4-byte aligned");
  return HISPARSE_OK;
}

// One decode call on checked arguments (batch > 0), for the layer pipeline
// optionally: with copy_layer >= 0 the same launch also copies that layer's
// misses (plan slice 0) in workgroups past the decode's own; its split
// partials go to half `half` of a two-half workspace; comb_out != nullptr
// combines the other half (the previous call of the same shape) into it in
// workgroups after the copy's; defer leaves this call's combine to the next
// launch.  A plain call (half -1) uses a one-half workspace.
static int decode_launch(hisparse_pool* pool, hipStream_t stream, int32_t batch, int32_t heads,
                         int32_t top_k, int32_t layer, const void* q_bf16,
                         const int32_t* device_buffer_locs, float softmax_scale, void* out_bf16,
                         int32_t copy_layer = -1, uint64_t* stats = nullptr, int half = -1,
                         void* comb_out = nullptr, bool defer = false) {
  const int splits = decode_splits(batch, heads, top_k);
  const size_t one = decode_workspace_bytes(batch, heads, splits);
  // Each half holds the largest shape the configuration admits (checked by
  // decode_check), so this is an internal invariant, not a caller error.
  const size_t half_bytes = pool->dec_ws_bytes / 2;
  if (one > half_bytes)
    return fail(HISPARSE_EUNSUPPORTED, "decode workspace of %zu bytes exceeds the pool's %zu", one,
                half_bytes);
  // each half: bf16 partial O, then fp32 (reference, denominator) per
  // (row, group, split, head)
  const size_t entries = one / (512 * sizeof(uint16_t) + 2 * sizeof(float));
  unsigned char* ws = (unsigned char*)pool->dec_ws;
  unsigned char* mine = ws + (half > 0 ? half_bytes : 0);
  DecodeParams d = {};
  d.splits = splits;
  d.part_o = (uint16_t*)mine;
  d.part_ml = (float*)(d.part_o + entries * 512);
  if (comb_out) {
    unsigned char* other = ws + (half > 0 ? 0 : half_bytes);
    d.comb_part_o = (const uint16_t*)other;
    d.comb_part_ml = (const float*)(d.comb_part_o + entries * 512);
    d.comb_out = (uint16_t*)comb_out;
  }
  d.defer_combine = defer ? 1 : 0;
  d.pool = pool->dev_ptrs[layer];
  d.pool_rows = pool->device_pool_rows;
  d.row_bytes = pool->cfg.row_bytes;
  d.heads = heads;
  d.k = top_k;
  d.batch = batch;
  d.scale = softmax_scale;
  d.q = (const uint16_t*)q_bf16;
  d.locs = device_buffer_locs;
  d.out = (uint16_t*)out_bf16;
  if (copy_layer >= 0) {
    d.copy_host = pool->host_ptrs[copy_layer];
    d.copy_dev = pool->dev_ptrs[copy_layer];
    d.copy_host_rows = pool->host_rows[copy_layer];
    d.plan_src = pool->plan_src;
    d.plan_dst = pool->plan_dst;
    d.plan_cnt = pool->plan_cnt;
    d.plan_stride = pool->cfg.max_top_k;
    d.units = pool->cfg.row_bytes / 16;
    d.stats = (unsigned long long*)stats;
  }
  hipError_t e = launch_sparse_mla_decode(d, batch, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse-MLA decode kernel launch");
  return HISPARSE_OK;
}

int hisparse_sparse_mla_decode(hisparse_pool* pool, void* stream, int32_t batch, int32_t heads,
                               int32_t top_k, int32_t layer, const void* q_bf16,
                               const int32_t* device_buffer_locs, float softmax_scale,
                               void* out_bf16) {
  int rc = decode_check(pool, batch, heads, top_k, layer, q_bf16, device_buffer_locs, out_bf16);
  if (rc != HISPARSE_OK) return rc;
  if (batch == 0) return ok();
  if ((rc = check_device(pool)) != HISPARSE_OK) return rc;
  rc = decode_launch(pool, (hipStream_t)stream, batch, heads, top_k, layer, q_bf16,
                     device_buffer_locs, softmax_scale, out_bf16);
  return rc == HISPARSE_OK ? ok() : rc;
}

int hisparse_decode_layers_overlapped(hisparse_pool* pool, void* stream, int32_t batch,
                                      int32_t heads, int32_t top_k, const void* const* q_bf16,
                                      const int32_t* device_buffer_locs, float softmax_scale,
                                      void* const* out_bf16, uint64_t* stats) {
  if (!pool) return fail(HISPARSE_EINVAL, "pool is NULL");
  if (!q_bf16 || !out_bf16) return fail(HISPARSE_EINVAL, "q_bf16 and out_bf16 must not be NULL");
  if (batch < 0 || batch > pool->cfg.max_batch)
    return fail(HISPARSE_EINVAL, "batch %d outside [0, max_batch=%d]", batch, pool->cfg.max_batch);
  if (stats && !aligned(stats, 8)) return fail(HISPARSE_EINVAL, "stats is not 8-byte aligned");
  if (batch == 0) return ok();
  const int L = pool->cfg.num_layers;
  int rc;
  for (int l = 0; l < L; ++l)  // every layer's arguments before anything is enqueued
    if ((rc = decode_check(pool, batch, heads, top_k, l, q_bf16[l], device_buffer_locs,
                           out_bf16[l])) != HISPARSE_OK)
      return rc;
  if ((rc = check_plan_batch(pool, batch, 0)) != HISPARSE_OK) return rc;
  if ((rc = check_device(pool)) != HISPARSE_OK) return rc;
  // All on the caller's stream, so no cross-stream events: layer 0's copy
  // alone, then one launch per layer that decodes layer l while its spare
  // workgroups copy layer l + 1 and combine layer l - 1's splits (each
  // launch reads only rows the one before it finished copying, and the
  // split partials of layers l and l - 1 sit in the two halves of the
  // workspace); the last layer's combine follows as its own kernel.
  hipStream_t us = (hipStream_t)stream;
  if ((rc = launch_copy(pool, us, batch, 0, 1, stats)) != HISPARSE_OK) return rc;
  for (int l = 0; l < L; ++l) {
    const bool last = l + 1 == L;
    rc = decode_launch(pool, us, batch, heads, top_k, l, q_bf16[l], device_buffer_locs,
                       softmax_scale, out_bf16[l], last ? -1 : l + 1, stats, l & 1,
                       l > 0 ? out_bf16[l - 1] : nullptr, !last);
    if (rc != HISPARSE_OK) return rc;
  }
  return ok();
}

int hisparse_sparse_mla_decode_noalloc(void* stream, int32_t batch, int32_t heads, int32_t top_k,
                                       const void* device_pool, int64_t device_pool_rows,
                                       int32_t row_bytes, const void* q_bf16,
                                       const int32_t* device_buffer_locs, float softmax_scale,
                                       void* out_bf16) {
  if (batch < 0) return fail(HISPARSE_EINVAL, "batch %d < 0", batch);
  if (heads <= 0 || heads % 16 != 0)
    return fail(HISPARSE_EUNSUPPORTED, "heads %d must be a positive multiple of 16", heads);
  if (top_k < 0 || top_k > kMaxTopK)
    return fail(HISPARSE_EINVAL, "top_k %d outside [0, %d]", top_k, kMaxTopK);
  if (row_bytes < 656 || row_bytes % 16 != 0)
    return fail(HISPARSE_EUNSUPPORTED, "row_bytes %d must be a multiple of 16 and >= 656", row_bytes);
  if (device_pool_rows < 0 || device_pool_rows > INT32_MAX)
    return fail(HISPARSE_EINVAL, "device_pool_rows outside [0, 2^31)");
  const int HG = (heads + 127) / 128;
  if ((int64_t)batch * HG > kNoAllocDecodeUnits)
    return fail(HISPARSE_EUNSUPPORTED,
                "batch %d x ceil(heads/128) = %lld exceeds the %d units of the static split "
                "workspace (%zu bytes)",
                batch, (long long)batch * HG, kNoAllocDecodeUnits,
                (size_t)kNoAllocDecodeUnits * kDecodeUnitBytes);
  if (batch == 0) return ok();
  if (!device_pool || !q_bf16 || !out_bf16 || (top_k > 0 && !device_buffer_locs))
    return fail(HISPARSE_EINVAL, "device_pool, q_bf16, out_bf16 and device_buffer_locs must not be NULL");
  if (!aligned(device_pool, 16) || !aligned(q_bf16, 16) || !aligned(out_bf16, 8) ||
      !aligned(device_buffer_locs, 4))
    return fail(HISPARSE_EINVAL,
                "device_pool and q_bf16 must be 16-byte, out_bf16 8-byte and locs 4-byte aligned");
  const int splits = decode_splits(batch, heads, top_k);
  const size_t one = decode_workspace_bytes(batch, heads, splits);
  if (one > (size_t)kNoAllocDecodeUnits * kDecodeUnitBytes)  // implied by the unit check above
    return fail(HISPARSE_EUNSUPPORTED, "decode workspace of %zu bytes exceeds the static one", one);
  void* ws = nullptr;
  int rc = noalloc_scratch(&ws);
  if (rc != HISPARSE_OK) return rc;
  const size_t entries = one / (512 * sizeof(uint16_t) + 2 * sizeof(float));
  DecodeParams d = {};
  d.splits = splits;
  d.part_o = (uint16_t*)ws;
  d.part_ml = (float*)(d.part_o + entries * 512);
  d.pool = (const unsigned char*)device_pool;
  d.pool_rows = device_pool_rows;
  d.row_bytes = row_bytes;
  d.heads = heads;
  d.k = top_k;
  d.batch = batch;
  d.scale = softmax_scale;
  d.q = (const uint16_t*)q_bf16;
  d.locs = device_buffer_locs;
  d.out = (uint16_t*)out_bf16;
  hipError_t e = launch_sparse_mla_decode(d, batch, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "sparse-MLA decode kernel launch");
  return ok();
}

}  // extern "C"
