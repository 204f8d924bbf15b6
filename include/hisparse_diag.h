/*
 * hisparse_diag.h -- diagnostic entry points of libhisparse_diag.so.
 *
 * libhisparse_diag.so is a second build of the same sources with the plan
 * kernel's phase trace compiled in, plus floor kernels of the plan kernel's
 * launch shape.  It exports every entry point of hisparse.h as well, so a
 * program runs unchanged on it; libhisparse.so exports none of the functions
 * below.  They exist to measure the plan kernel, whose phases are the
 * resolver phases of "vLLM Hybrid HiSparse 源码实现分析" section 7.2 (hit
 * detection, LRU refresh, victim choice, plan emission).
 *
 * Status codes are those of hisparse.h; hisparse_last_error() gives the
 * message of the last failure.
 */
#ifndef HISPARSE_DIAG_H
#define HISPARSE_DIAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shape of the phase trace: [rows][waves][points][2] of uint64. */
#define HISPARSE_TRACE_ROWS 256  /* batch rows traced (rows 0 .. 255)         */
#define HISPARSE_TRACE_WAVES 16  /* wavefronts of a plan workgroup           */
#define HISPARSE_TRACE_POINTS 9  /* points 0-7 below, then point 8 (info)    */
#define HISPARSE_TRACE_WORDS                                                  \
  (HISPARSE_TRACE_ROWS * HISPARSE_TRACE_WAVES * HISPARSE_TRACE_POINTS * 2)

/*
 * Phase trace of the plan kernel (both its plan-only and its fused plan +
 * copy instances).  Lane 0 of every wavefront of a traced batch row stores,
 * at each point, [0] the shader clock (s_memtime) and [1] the 100 MHz
 * real-time counter:
 *   0 kernel entry;
 *   1 the request's loads issued and the LDS table cleared (first barrier);
 *   2 validity, resident pages and table inserts done (step 1);
 *   3 every slot probed the table, hit slots chosen (step 2);
 *   4 hits, misses and the per-wave partials done (step 3);
 *   5 victims ranked (step 4: windows, or the sort fallback);
 *   6 plan, row IDs and slot state written (step 5);
 *   7 end of the workgroup (after the fused copy in the fused instance).
 * Point 8 holds [0] the ranking windows used (0: no miss, or the row's
 * smallest key alone covered every miss) and [1] 1 if the sort fallback
 * ran.  Rows that take the fast path (seq_len <= slots) or are padding
 * return after point 0.  The trace of a launch overwrites the one before;
 * points a launch does not reach keep what was there, so clear between
 * launches.
 */

/* Zeroes the trace (synchronous: waits for the device).  Returns HISPARSE_OK
 * or HISPARSE_EHIP. */
int hisparse_diag_phase_clear(void);

/* Copies the trace to `host_out` (count = HISPARSE_TRACE_WORDS uint64,
 * layout [row][wave][point][2]) after waiting for the device.  Returns
 * HISPARSE_EINVAL for a null pointer or another count, HISPARSE_EHIP if the
 * copy fails. */
int hisparse_diag_phase_read(uint64_t* host_out, size_t count);

/*
 * Floor kernels of the plan kernel's launch shape: `batch` workgroups of
 * 1024 threads, one per batch row, on `stream`.  Device pointers, row-major,
 * as hisparse_resolve takes them.  `kind`:
 *   0 an empty kernel (only `batch` is read);
 *   1 one global round trip: req_idx[b] stored to out[b][0 .. top_k);
 *   2 two dependent round trips: req_idx[b], then that request's slot map
 *     and stamps (slots int32 each, coalesced), reduced and stored to
 *     out[b][..];
 *   3 the plan's memory chain without its computation: top-k row and
 *     req_idx[b]; then slot map and stamps; a workgroup exchange (a miss is
 *     known only once every slot has been seen); then host_cache_locs at
 *     every entry's position (dependent on the slot data); out[b][i] = the
 *     low 32 bits of that location.
 * Request rows are clamped to [0, max_requests), positions to
 * [0, max_seq_len), so every access stays inside the arrays; `out`
 * ([batch][top_k] int32) is scratch of the caller.  The kernel is launched
 * `launches` times back to back (1 <= launches <= 1048576), so that events
 * around one call time the kernels, not the caller's loop.  Returns
 * HISPARSE_EINVAL for a bad kind, size or null pointer the kind reads
 * (1 <= batch <= 65535, 1 <= top_k <= 4096, 1 <= slots <= 16384),
 * HISPARSE_EHIP if a launch fails.
 */
int hisparse_diag_floor(void* stream, int32_t kind, int32_t batch, int32_t top_k, int32_t slots,
                        int32_t max_requests, int64_t max_seq_len, const int32_t* req_idx,
                        const int32_t* top_k_tokens, const int32_t* slot_tokens,
                        const int32_t* lru_slots, const int64_t* host_cache_locs, int32_t* out,
                        int32_t launches);

/*
 * Hit detection alone, both ways round, for a measured comparison: one
 * 1024-thread workgroup per batch row on `stream`.
 * out[b][i] (int32 [batch][top_k]) = the lowest slot s of request
 * req_idx[b] (clamped to [0, max_requests)) with slot_tokens[r][s] equal to
 * entry i's position, or -1 (also for positions outside
 * [0, min(seq_lens[b], max_seq_len))).  `mode`:
 *   0 the entries' positions go into an LDS table and every slot probes it
 *     with its token (the plan kernel's direction);
 *   1 the slots' tokens go into an LDS table (a slot -> token map, lowest
 *     slot per token) and every entry probes it with its position;
 *   2, 3 the same two directions with the plan kernel's kind of table:
 *     buckets of 4 cells filled in order through a fill count per bucket
 *     and read 16 bytes at a time; 8 cells per entry for 2 (4 at
 *     top_k = 4096), 4 per slot for 3.
 * Modes 0 and 1 use single-cell linear probing, 4 cells per inserted item.
 * Positions within a row must be distinct, as for hisparse_resolve.
 * Launched `launches` times back to back.  Returns HISPARSE_EINVAL for a bad
 * mode, a NULL array, 1 <= batch <= 65535, 1 <= top_k <= 4096,
 * 1 <= slots <= 4096, max_requests or max_seq_len < 1, or launches outside
 * [1, 1048576]; HISPARSE_EHIP if a launch fails.
 */
int hisparse_diag_hit_detection(void* stream, int32_t mode, int32_t batch, int32_t top_k,
                                int32_t slots, int32_t max_requests, int64_t max_seq_len,
                                const int32_t* req_idx, const int32_t* top_k_tokens,
                                const int32_t* seq_lens, const int32_t* slot_tokens, int32_t* out,
                                int32_t launches);

/*
 * The cost of splitting one request over several workgroups: `groups`
 * workgroups of 256 threads per batch row (grid batch * groups), where each
 * writes 64 ints of partials, makes them visible device-wide (agent-scope
 * fence), and bumps its row's arrival counter; the last to arrive reads
 * every partial of the row, stores their per-thread sums and resets the
 * counter.  No workgroup waits for another.  `scratch` is device int32
 * [batch][HISPARSE_EXCHANGE_ROW_INTS]: [0] the arrival counter (zero before
 * the first call; each call leaves it zero), [32, 64) the sums, [64, ...)
 * the partials.  Launched `launches` times back to back.  Returns
 * HISPARSE_EINVAL for a null scratch, 1 <= batch * groups <= 65535 or
 * 1 <= groups <= 16 violated, or launches outside [1, 1048576];
 * HISPARSE_EHIP if a launch fails.
 */
#define HISPARSE_EXCHANGE_ROW_INTS (64 + 64 * 16)
int hisparse_diag_exchange(void* stream, int32_t batch, int32_t groups, int32_t* scratch,
                           int32_t launches);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_DIAG_H */
