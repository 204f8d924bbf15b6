/*
 * hisparse.h -- C ABI of the HiSparse swap-in resolver for AMD Instinct
 * MI355X (gfx950).
 *
 * On each decode step the resolver takes every batch row's top-k token
 * positions (chosen by the model's sparse-attention indexer) and turns them
 * into physical device row IDs that sparse-MLA decode attention reads:
 *   1. positions in resident device pages resolve in place;
 *   2. positions already in the request's fixed-size hot buffer are hits and
 *      get their LRU stamp refreshed;
 *   3. the remaining positions (misses) take LRU victim slots;
 *   4. the missing KV rows are copied from pinned host memory into those
 *      slots (once per layer that shares the index);
 *   5. the row IDs are written to device_buffer_locs.
 * This is the fused resolver of "vLLM HiSparse 本地 KV 卸载架构" (section on
 * hot-row lookup and LRU: resident page -> hot row + LRU refresh -> LRU victim
 * + pinned host copy) and the swap-in kernel of the SGLang HiSparse pages
 * ("HiSparse: 把长上下文 decode 的容量瓶颈从 GPU 显存搬到 CPU 内存", section
 * "Core: the swap-in CUDA kernel", whose parameters are lru_slots,
 * host_cache_locs, device_buffer_locs, top_k_tokens and seq_lens).
 *
 * Conventions for every entry point:
 *  - Status codes are returned synchronously; nothing throws across the ABI.
 *    On a non-OK return hisparse_last_error() holds a message (per thread).
 *  - "device" pointers are HIP device memory (e.g. torch CUDA tensors);
 *    "host" pointers are ordinary host memory.  The caller owns every buffer
 *    it passes and keeps it alive while the pool uses it.
 *  - Work is enqueued on the given stream (a hipStream_t passed as void*;
 *    NULL = the null stream).  No entry point that takes a stream
 *    synchronises the device or reads device memory back to the host, so the
 *    calls are stream-ordered and can be captured in a HIP graph.
 *  - Calls that share one pool must be ordered (one stream, or explicit
 *    events): the pool's miss-plan workspace is shared by all of them.
 *  - Anomalies found on the device (corrupt state, out-of-range host rows)
 *    never abort: they follow the documented tripwire rules and are counted
 *    in stats[4].
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  HISPARSE_OK = 0,
  HISPARSE_EINVAL = -1,      /* bad argument (checked on the host)           */
  HISPARSE_ENOMEM = -2,      /* allocation or pinning failed                 */
  HISPARSE_EHIP = -3,        /* a HIP runtime call or kernel launch failed   */
  HISPARSE_EUNSUPPORTED = -4 /* shape outside what the kernels support       */
};

/* Indices into the optional uint64 stats[5] device array (accumulated with
 * atomic adds, never read back by the library).  The hit/miss pair mirrors
 * the swap statistics of "vLLM Hybrid HiSparse 源码实现分析" section 7.1. */
enum {
  HISPARSE_STAT_HOT_HITS = 0,
  HISPARSE_STAT_MISSES = 1,
  HISPARSE_STAT_RESIDENT_HITS = 2,
  HISPARSE_STAT_FAST_PATH = 3,
  HISPARSE_STAT_TRIPWIRES = 4
};

typedef struct hisparse_pool hisparse_pool; /* opaque, library-owned */

typedef struct {
  int32_t max_requests;   /* R: request-state rows                              */
  int32_t slots;          /* S: hot slots per request (device_buffer_size),
                             1..16384                                           */
  int32_t max_top_k;      /* largest top_k of any call, 1..S and <= 4096.  The
                             resolver keeps one request's table in 160 KB of
                             LDS, about max(7*pow2(8k) + 4k, 8*pow2(S)) + 16k
                             bytes (the table drops to 4, then 2, cells per
                             entry when 8 do not fit); init returns
                             EUNSUPPORTED for a pair that does not fit.
                             k=2048 needs 153 KB at S=4096 and at S=6144;
                             S <= 8192 allows k up to 4096, S=16384 up to
                             2004.                                              */
  int32_t max_batch;      /* largest batch of any call (sizes the miss plan),
                             1..65535                                           */
  int32_t row_bytes;      /* bytes per KV row, a multiple of 16 (656 for the
                             fp8 sparse-MLA row)                                 */
  int32_t num_layers;     /* L >= 1 layers that share one index and one plan    */
  int32_t page_size;      /* P: tokens per resident page; 0 = no resident tier  */
  int32_t max_steps;      /* verification steps per hisparse_resolve_steps call
                             (speculative decoding); 0 or 1 = one.  The miss
                             plan workspace holds this many slices.             */
  int32_t max_heads;      /* largest `heads` of any decode call (a multiple of
                             16), or 0 if the pool never decodes.  Sizes the
                             decode's split workspace, allocated at init:
                             2 * max(256, max_batch * ceil(max_heads/128))
                             * 132096 bytes (67.6 MB at max_batch <= 256 and
                             max_heads <= 128).                                 */
  int64_t resident_pages; /* resident pages in each device pool (0 if P == 0)   */
  int64_t max_seq_len;    /* row stride, in tokens, of host_cache_locs and
                             (divided by P, rounded up) of the block table      */
} hisparse_pool_config;

/*
 * hisparse_host_alloc / hisparse_host_free
 *   Allocate `bytes` of pinned host memory that kernels can read directly
 *   (the host tier: "pinned host pool" of the vLLM HiSparse architecture
 *   page, ownership table).  The memory is page-locked, mapped into the
 *   device address space, and 4096-byte aligned.  Host pools given to
 *   hisparse_init_pool must come from here (or from another hipHostMalloc).
 *   A request above 95% of the host's available memory (MemAvailable in
 *   /proc/meminfo) is refused with ENOMEM before anything is pinned, as the
 *   worker of "vLLM Hybrid HiSparse 源码实现分析" (section 2.4) refuses to
 *   start when the host pool would not fit in RAM; pinning nearly all of RAM
 *   would leave the host to the out-of-memory killer.  Returns ENOMEM if the
 *   allocation fails.  hisparse_host_free(NULL) is a no-op.
 */
int hisparse_host_alloc(size_t bytes, void** out);
int hisparse_host_free(void* ptr);

/*
 * hisparse_init_pool
 *   host_pools[L]      host: pinned host pool of layer l, host_pool_rows[l]
 *                      rows of row_bytes each (rows addressed by
 *                      host_cache_locs).
 *   host_pool_rows[L]  host: row counts of the host pools, each < 2^31
 *                      (1.4 TB of 656-byte rows per layer).
 *   device_pools[L]    device: one row pool per layer, device_pool_rows rows of
 *                      row_bytes, 16-byte aligned.  Resident and hot rows share
 *                      it ("vLLM Hybrid HiSparse 源码实现分析" section 2.2):
 *                        hot row of (request r, slot s)     = r*S + s
 *                        resident row of (page p, offset o) = R*S + p*P + o
 *   device_pool_rows   >= R*S + resident_pages*P and < 2^31.
 *   out                receives the pool.  The pool allocates its miss-plan
 *                      workspace in device memory (12 bytes per
 *                      max_batch*max_top_k entry per plan slice) and, when
 *                      max_heads > 0, the decode's split workspace; it frees
 *                      both on destroy.  No later call allocates.
 *   Errors: EINVAL (shape, alignment, a host pool that is not pinned,
 *   max_heads not a multiple of 16), ENOMEM, EHIP.  Must be called with the
 *   target device current.
 */
int hisparse_init_pool(const hisparse_pool_config* config,
                       void* const* host_pools, const int64_t* host_pool_rows,
                       void* const* device_pools, int64_t device_pool_rows,
                       hisparse_pool** out);

/*
 * hisparse_resolve -- one decode step: plan (steps 1-3 and 5 above) then the
 * miss copy into all L layers (step 4).  Equivalent to hisparse_resolve_plan
 * followed by hisparse_gather_copy(pool, stream, batch, 0, L, stats).
 *
 * All arrays are device memory, row-major, int32 unless stated:
 *   req_idx[batch]                 request-state row of each batch row;
 *                                  < 0 = padding row (all outputs -1);
 *                                  >= R is treated as padding and counts one
 *                                  tripwire.  Active rows must be distinct.
 *   top_k_tokens[batch][top_k]     logical positions; an entry outside
 *                                  [0, min(seq_len, max_seq_len)) is invalid:
 *                                  output -1, no state change.  Valid entries
 *                                  of one row must be distinct (otherwise the
 *                                  result is unspecified but memory-safe).
 *   seq_lens[batch]                current sequence length of each row.
 *   host_cache_locs[R][max_seq_len] int64 host row of every token.  A value
 *                                  outside [0, host_pool_rows[l]) zero-fills
 *                                  the destination row of layer l and counts
 *                                  one tripwire.
 *   resident_block_table[R][ceil(max_seq_len/P)]  physical resident page of
 *                                  each logical page, < 0 = not resident;
 *                                  may be NULL.  An id >= resident_pages is
 *                                  treated as not resident (one tripwire).
 *   slot_tokens[R][S]              state: token held by each hot slot, -1 =
 *                                  empty (values < -1 also count as empty).
 *   lru_slots[R][S]                state: last-use stamp of each slot.
 *   lru_clock[R]                   state: per-request clock, +1 per call in
 *                                  which the row is active.
 *   device_buffer_locs[batch][top_k]  output row IDs (-1 = none).
 *   stats[5]                       uint64 counters (see above), or NULL.
 * Initial state: slot_tokens all -1, lru_slots all 0, lru_clock all 0.
 *
 * Per active row (r = req_idx[b], n = seq_lens[b], c = ++lru_clock[r]):
 *  - Fast path, n <= S ("HiSparse: 把长上下文 decode ..." page, flow of each
 *    decode step: a sequence that fits the buffer is already in it): every
 *    valid t gives r*S + t, sets slot_tokens[r][t] = t and lru_slots[r][t] = c;
 *    nothing is copied.  The caller keeps device row r*S+t filled with token t.
 *  - Otherwise ("vLLM Hybrid HiSparse 源码实现分析" section 7.2):
 *    resident entries resolve in place; then each remaining t held by a slot
 *    is a hit (lowest such slot) and refreshes that slot's stamp to c; the
 *    misses, in ascending top-k index, take the non-hit slots in ascending
 *    (occupied, stamp, slot) order -- empty first, then least recently used,
 *    ties by lowest slot -- and become slot_tokens = t, stamp c, with
 *    host_cache_locs[r][t] copied into that row of every layer.
 * Host-side checks (EINVAL): null required pointer, misaligned pointer,
 * batch > max_batch, top_k > max_top_k.
 */
int hisparse_resolve(hisparse_pool* pool, void* stream, int32_t batch,
                     int32_t top_k, const int32_t* req_idx,
                     const int32_t* top_k_tokens, const int32_t* seq_lens,
                     const int64_t* host_cache_locs,
                     const int32_t* resident_block_table, int32_t* slot_tokens,
                     int32_t* lru_slots, int32_t* lru_clock,
                     int32_t* device_buffer_locs, uint64_t* stats);

/*
 * hisparse_resolve_plan -- hisparse_resolve without the copy: resolves every
 * entry, updates the state and writes device_buffer_locs, and stores the miss
 * plan (host row, device row) of each batch row in the pool's workspace.
 * Same arguments and checks as hisparse_resolve.
 */
int hisparse_resolve_plan(hisparse_pool* pool, void* stream, int32_t batch,
                          int32_t top_k, const int32_t* req_idx,
                          const int32_t* top_k_tokens, const int32_t* seq_lens,
                          const int64_t* host_cache_locs,
                          const int32_t* resident_block_table,
                          int32_t* slot_tokens, int32_t* lru_slots,
                          int32_t* lru_clock, int32_t* device_buffer_locs,
                          uint64_t* stats);

/*
 * hisparse_gather_copy -- copy the rows of the last plan into the device
 * pools of layers [layer_begin, layer_end).  Layers that share one index
 * replay the same plan and copy only their own bytes ("vLLM Hybrid HiSparse
 * 源码实现分析" section 7.4, follower layers).  `batch` must equal the batch
 * of the last plan enqueued on this pool (checked on the host: a different
 * batch would replay rows of an older plan).  stats may be NULL (tripwires
 * are then not counted).
 * Errors: EINVAL for a layer range outside [0, L), a batch other than the
 * plan's, or no plan yet.
 */
int hisparse_gather_copy(hisparse_pool* pool, void* stream, int32_t batch,
                         int32_t layer_begin, int32_t layer_end,
                         uint64_t* stats);

/*
 * hisparse_sparse_mla_decode -- decode attention of one layer over the rows
 * named by device_buffer_locs (the consumer of the row IDs: "vLLM HiSparse
 * 本地 KV 卸载架构", ownership table: the attention backend consumes the
 * device cache and physical row IDs).  Row format ("vLLM Hybrid HiSparse
 * 源码实现分析" section 9): bytes 0..511 latent in fp8 e4m3 (OCP), bytes
 * 512..527 four fp32 scales (one per 128 latent values), bytes 528..655 the
 * 64-value bf16 rope part.  For each batch row b and head h:
 *   K_i = [e4m3(latent_i) * scale ; rope_i] (576), V_i = e4m3(latent_i)*scale
 *   O[b][h] = softmax_i(softmax_scale * q[b][h] . K_i) V_i over entries with
 *   0 <= loc < device_pool_rows (O = 0 if there are none).
 *   q_bf16   device bf16 [batch][heads][576]
 *   out_bf16 device bf16 [batch][heads][512]
 * Requires row_bytes >= 656, heads a multiple of 16 and <= max_heads,
 * batch <= max_batch, top_k <= max_top_k.  The keys of each row are split
 * across workgroups and a second kernel combines the partial results, in
 * the pool's split workspace sized at init (see max_heads): the call
 * allocates nothing and never synchronises.  Calls on one pool that overlap
 * in time (different streams) race on this workspace.  A NaN in a row that
 * is attended to (a 0x7F/0xFF latent code, a NaN scale) makes that row's
 * outputs NaN, as the softmax of a NaN score is.  Errors: EINVAL,
 * EUNSUPPORTED, EHIP.
 */
int hisparse_sparse_mla_decode(hisparse_pool* pool, void* stream,
                               int32_t batch, int32_t heads, int32_t top_k,
                               int32_t layer, const void* q_bf16,
                               const int32_t* device_buffer_locs,
                               float softmax_scale, void* out_bf16);

/*
 * hisparse_resolve_steps -- the verification steps of speculative decoding
 * (multi-token prediction): `steps` resolver steps in order, each exactly
 * hisparse_resolve on its own slice of the arguments, with step q planned
 * into plan slice q of the workspace (replayable with
 * hisparse_gather_copy_step) and all steps sharing the requests' hot state
 * ("vLLM Hybrid HiSparse 源码实现分析" section 7.4; the architecture page's
 * note on speculative decoding).
 *   top_k_tokens        [steps][batch][top_k]
 *   seq_lens            [steps][batch]
 *   device_buffer_locs  [steps][batch][top_k] (out)
 * Requires steps <= max(1, config.max_steps) and steps * top_k <= slots:
 * then every victim of step q is older than this call, so no step evicts a
 * row that an earlier step of the same call returned (the page's hot
 * region of (query length + 1) * top_k rows meets this with one top_k to
 * spare).  Errors: as hisparse_resolve, and EINVAL for the two bounds.
 */
int hisparse_resolve_steps(hisparse_pool* pool, void* stream, int32_t steps, int32_t batch,
                           int32_t top_k, const int32_t* req_idx, const int32_t* top_k_tokens,
                           const int32_t* seq_lens, const int64_t* host_cache_locs,
                           const int32_t* resident_block_table, int32_t* slot_tokens,
                           int32_t* lru_slots, int32_t* lru_clock, int32_t* device_buffer_locs,
                           uint64_t* stats);

/* hisparse_gather_copy_step -- hisparse_gather_copy of plan slice `step`
 * (0 <= step < max(1, max_steps)), e.g. for the follower layers of one
 * verification step.  Errors: EINVAL, EHIP. */
int hisparse_gather_copy_step(hisparse_pool* pool, void* stream, int32_t step, int32_t batch,
                              int32_t layer_begin, int32_t layer_end, uint64_t* stats);

/*
 * hisparse_mirror_rows -- the row mirror (eager backup): copy device rows
 * back to their host rows in layers [layer_begin, layer_end):
 *   host_pool[l][host_rows[i]] = device_pool[l][dev_rows[i]], i < count.
 * This is the last step of a decode step in the per-step flow of the
 * gogongxt.com HiSparse page (the previous token's row goes back to the
 * host), and the row mirror of "vLLM Hybrid HiSparse 源码实现分析" section 6
 * (rows written by the forward pass are mirrored so that a later spill
 * moves no data).  It keeps "every token t < seq_len has its host row" true
 * in a running decode loop.
 *   dev_rows[count]   device int32: device pool rows; < 0 = padding entry
 *                     (skipped, not counted)
 *   host_rows[count]  device int64: destination host rows
 *   stats             device uint64[5] or NULL: stats[4] += 1 per layer for
 *                     a device row >= device_pool_rows or a host row
 *                     outside [0, host_pool_rows[l]) (that copy is skipped)
 * Destinations must be distinct (if not, which copy lands is unspecified;
 * memory stays safe).  Stream-ordered, no readback.  Errors: EINVAL, EHIP.
 */
int hisparse_mirror_rows(hisparse_pool* pool, void* stream, int32_t count,
                         const int32_t* dev_rows, const int64_t* host_rows,
                         int32_t layer_begin, int32_t layer_end, uint64_t* stats);

/*
 * hisparse_invalidate_tokens -- for each entry i < count, empty every hot
 * slot of request row req_rows[i] holding a token in
 * [tok_begin[i], tok_end[i]): slot_tokens = -1, lru_slots = 0 (the state of
 * a never-used slot, first in victim order).  The precise clearing of rows
 * rewritten by a prefill ("vLLM Hybrid HiSparse 源码实现分析" section 6, hot-
 * cache coherence); with [0, INT32_MAX) it clears a request row that is
 * handed to a new request.  All arrays are device int32 of length count
 * except the state ([R][S]).  req_rows[i] < 0 is padding; >= R counts one
 * tripwire in stats[4] (stats may be NULL).  Errors: EINVAL, EHIP.
 */
int hisparse_invalidate_tokens(hisparse_pool* pool, void* stream, int32_t count,
                               const int32_t* req_rows, const int32_t* tok_begin,
                               const int32_t* tok_end, int32_t* slot_tokens,
                               int32_t* lru_slots, uint64_t* stats);

/*
 * hisparse_invalidate_host_rows -- empty every hot slot, of every request
 * row, whose token t maps to a host row host_cache_locs[r][t] in the set
 * rows_sorted[count] (device int64, ascending): host rows that were reused
 * for other content or rewritten ("vLLM Hybrid HiSparse 源码实现分析"
 * section 6: newly allocated host blocks are matched in a batch against
 * the hot entries).  Slots with tokens outside [0, max_seq_len) are left
 * alone.  The set is binary-searched, in LDS when it holds at most 8192
 * rows; an unsorted set gives an unspecified (memory-safe) result.
 * Errors: EINVAL, EHIP.
 */
int hisparse_invalidate_host_rows(hisparse_pool* pool, void* stream, int32_t count,
                                  const int64_t* rows_sorted, const int64_t* host_cache_locs,
                                  int32_t* slot_tokens, int32_t* lru_slots);

/*
 * hisparse_decode_layers_overlapped -- the miss copy and the decode of every
 * layer, pipelined: after a plan (hisparse_resolve_plan, or slice 0 of
 * hisparse_resolve_steps) enqueued on `stream`, layer 0's misses are copied,
 * then each layer's decode runs in one launch with the copy of the next
 * layer's misses and the split combine of the previous layer, so the copy
 * of layer l+1 overlaps the attention of layer l.  This is the layer-group pipelining of "vLLM Hybrid HiSparse 源码实现分析"
 * section 6 (each group is submitted when ready) on the swap-in side.
 * Everything is enqueued on `stream` alone, in stream order (no other
 * streams or events).  Results are those of hisparse_gather_copy of all
 * layers followed by hisparse_sparse_mla_decode of each layer l with
 * q_bf16[l] and out_bf16[l] (host arrays of L device pointers); stats[4]
 * counts the copy's tripwires.  The split partials of consecutive layers
 * use the two halves of the workspace sized at init, so nothing is
 * allocated.  Every layer's arguments, and that batch equals the plan's,
 * are checked before anything is enqueued.  Errors: as those calls.
 */
int hisparse_decode_layers_overlapped(hisparse_pool* pool, void* stream, int32_t batch,
                                      int32_t heads, int32_t top_k, const void* const* q_bf16,
                                      const int32_t* device_buffer_locs, float softmax_scale,
                                      void* const* out_bf16, uint64_t* stats);

/*
 * hisparse_sparse_mla_decode_noalloc -- hisparse_sparse_mla_decode without a
 * pool and without allocating anything, for callers that cannot allocate
 * device memory: code under stream capture set up before any pool exists,
 * serving loops and harnesses that forbid hipMalloc.  Same attention, same
 * kernels and key splits, so its output equals hisparse_sparse_mla_decode's
 * bit for bit on the same rows.
 *   device_pool       device: one layer's rows, device_pool_rows rows of
 *                     row_bytes (>= 656, a multiple of 16), 16-byte aligned
 *   q_bf16, device_buffer_locs, softmax_scale, out_bf16: as in
 *                     hisparse_sparse_mla_decode
 * The split partials live in a static device array of the library (33.8 MB,
 * held on every GPU the library runs on until the process ends), so
 * batch * ceil(heads / 128) must not exceed 256 (EUNSUPPORTED otherwise);
 * heads is a multiple of 16 and top_k <= 4096.  The array's address is
 * looked up on the first call on each device.  Every call on one GPU shares
 * that array: calls that overlap in time on one GPU (different streams, or
 * different threads) race on it and must be ordered by the caller.  Errors:
 * EINVAL, EUNSUPPORTED, EHIP.
 */
int hisparse_sparse_mla_decode_noalloc(void* stream, int32_t batch, int32_t heads, int32_t top_k,
                                       const void* device_pool, int64_t device_pool_rows,
                                       int32_t row_bytes, const void* q_bf16,
                                       const int32_t* device_buffer_locs, float softmax_scale,
                                       void* out_bf16);

/* Free the pool's workspace and the pool.  NULL is a no-op.  The caller must
 * make sure no work that uses the pool is still queued. */
void hisparse_destroy_pool(hisparse_pool* pool);

/* Message of the last non-OK return on this thread ("" if none). */
const char* hisparse_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
