/*
 * hisparse_oracle.c -- plain, single-threaded CPU oracle of the HiSparse
 * swap-in resolver and of the sparse-MLA decode step that consumes it.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this file; only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it (through oracle/oracle.py).  It shares no code,
 * header or constant with the HIP library: every definition below is written
 * out again from the pages.
 *
 * Sources (page titles as published; section names glossed in English):
 *  [P1] "vLLM HiSparse 本地 KV 卸载架构" (vLLM HiSparse local KV offload
 *       architecture), sections "Hot-row lookup and LRU", "Performance
 *       invariants", and the appended LMSYS blog section "An efficient
 *       swap-in kernel".
 *  [P2] "HiSparse: 把长上下文 decode 的容量瓶颈从 GPU 显存搬到 CPU 内存"
 *       (gogongxt.com), sections "The flow of each decode step" and
 *       "Core: the swap-in CUDA kernel".
 *  [P3] "vLLM Hybrid HiSparse 源码实现分析" (vLLM Hybrid HiSparse source
 *       analysis), sections 7.1 (data structures), 7.2 (the resolve kernel
 *       phase by phase), 7.3 (output is an HMA row ID), 7.4 (IndexShare),
 *       9 (the 656-byte fp8 row).
 *  [P4] "分层稀疏注意力框架下的 KV 分层管理与按需加载" (Alibaba Tair KVCache
 *       hierarchical sparse attention), section 2.4.3 (Sparse Diff Kernel).
 *  [P5] "vLLM GLM 5.3 优化：Hybrid HiSparse Offloading", section
 *       "2. Mixed Residency".
 *
 * Readings of points the pages leave open (each is also listed in the
 * design notes of the repository):
 *  - LRU state is one int32 stamp per slot plus one int32 clock per request
 *    row; a row's clock is bumped once per call in which the row is active,
 *    and every slot the call touches gets the new clock value.
 *  - Victim order: empty slots first, then the oldest stamp, ties broken by
 *    ascending slot index; misses are taken in ascending top-k index.
 *  - A hot slot is keyed by the logical token position inside its request.
 *  - Fast path when seq_len <= slots (inclusive); slot index == position.
 *  - A slot whose token is < -1 counts as empty; if (after corruption)
 *    several slots hold one position, the lowest slot index is the hit.
 *  - Entries outside [0, min(seq_len, max_seq_len)) are invalid: they give
 *    -1, are not counted and change no state.
 *  - A request index outside [0, R) makes the batch row a padding row; an
 *    index >= R also counts one tripwire.
 *  - A block-table entry >= resident_pages is treated as not resident and
 *    counts one tripwire.
 *  - A host row outside [0, host_pool_rows[l]) zero-fills the destination
 *    row of layer l and counts one tripwire.
 *
 * parity pinned: see tests/test_oracle_pins.py (LRU-cache reduction, set
 * counts, exhaustive tiny cases against an independent formulation,
 * invariants, fp8/bf16 decode against the torch CPU codecs, attention
 * against torch's CPU float64 attention).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)
#define OR_ENOMEM (-2)

/* Statistics slots, in order: hot hits, misses, resident hits, fast-path
 * rows, tripwires (counter layout of [P3] 7.1 extended by three fields). */
enum { ST_HITS = 0, ST_MISSES = 1, ST_RESIDENT = 2, ST_FAST = 3, ST_TRIP = 4 };

typedef struct {
  int32_t occupied; /* 1 if the slot holds a token, 0 if empty */
  int32_t stamp;    /* last-use clock value */
  int32_t slot;     /* slot index */
} victim_key;

/* Victim order of a non-hit slot: (occupied, stamp, slot) ascending, i.e.
 * empty first, then least recently used, then lowest slot index. */
static int cmp_victim(const void* a, const void* b) {
  const victim_key* x = (const victim_key*)a;
  const victim_key* y = (const victim_key*)b;
  if (x->occupied != y->occupied) return x->occupied < y->occupied ? -1 : 1;
  if (x->stamp != y->stamp) return x->stamp < y->stamp ? -1 : 1;
  if (x->slot != y->slot) return x->slot < y->slot ? -1 : 1;
  return 0;
}

/*
 * oracle_resolve: one decode step of the resolver for `batch` rows.
 *
 * Follows [P1] "Hot-row lookup and LRU" (resident page -> hot row with an
 * LRU refresh -> LRU victim plus a pinned-host row copy), [P3] 7.2 phases
 * 1-4 (resident short-circuit, hit classification, miss plan with victim
 * choice, LRU rewrite), [P2] "The flow of each decode step" (fast path when
 * seq_len <= device buffer size: nothing moves), [P3] 7.3 (row IDs shared by
 * resident and hot rows) and [P3] 7.4 (every layer that shares the index
 * receives the same slot assignment, bytes copied per layer).
 *
 * Device row space (one pool per layer, resident and hot rows share it):
 *   hot row of (r, s)          = r * S + s
 *   resident row of (page p, o) = R * S + p * P + o
 *
 * Arrays (row-major):
 *   req_idx[batch], top_k_tokens[batch][top_k], seq_lens[batch]
 *   host_cache_locs[R][max_seq_len] (int64 host row per token)
 *   block_table[R][ceil(max_seq_len / P)] or NULL
 *   slot_tokens[R][S], lru_slots[R][S], lru_clock[R]   (state, in/out)
 *   out[batch][top_k]                                   (row IDs, -1 = none)
 *   stats[5]                                            (accumulated)
 *   host_pools[L] -> rows of row_bytes; dev_pools[L] -> dev_pool_rows rows
 *
 * When `validate` is non-zero the call first rejects precondition
 * violations (duplicate valid positions in one row, one request index on
 * two active rows) with OR_EINVAL and changes nothing.
 */
int oracle_resolve(int32_t R, int32_t S, int32_t row_bytes, int32_t L,
                   int32_t P, int64_t max_seq_len, int64_t resident_pages,
                   int32_t batch, int32_t top_k, const int32_t* req_idx,
                   const int32_t* top_k_tokens, const int32_t* seq_lens,
                   const int64_t* host_cache_locs, const int32_t* block_table,
                   int32_t* slot_tokens, int32_t* lru_slots,
                   int32_t* lru_clock, int32_t* out, uint64_t* stats,
                   uint8_t* const* host_pools, const int64_t* host_pool_rows,
                   uint8_t* const* dev_pools, int64_t dev_pool_rows,
                   int validate) {
  int64_t max_pages = 0;
  if (P > 0) max_pages = (max_seq_len + P - 1) / P;
  if (R <= 0 || S <= 0 || batch < 0 || top_k < 0 || top_k > S || L <= 0 ||
      row_bytes <= 0)
    return OR_EINVAL;
  if ((int64_t)R * S + resident_pages * (int64_t)(P > 0 ? P : 0) >
      dev_pool_rows)
    return OR_EINVAL;

  if (validate) {
    /* Preconditions: distinct valid positions per row; distinct requests. */
    for (int32_t b = 0; b < batch; ++b) {
      int32_t r = req_idx[b];
      if (r < 0 || r >= R) continue;
      for (int32_t b2 = b + 1; b2 < batch; ++b2)
        if (req_idx[b2] == r) return OR_EINVAL;
      int64_t n = seq_lens[b];
      if (n > max_seq_len) n = max_seq_len;
      const int32_t* row = top_k_tokens + (int64_t)b * top_k;
      for (int32_t i = 0; i < top_k; ++i) {
        if (row[i] < 0 || row[i] >= n) continue;
        for (int32_t i2 = i + 1; i2 < top_k; ++i2)
          if (row[i2] == row[i]) return OR_EINVAL;
      }
    }
  }

  victim_key* keys = (victim_key*)malloc(sizeof(victim_key) * (size_t)S);
  int32_t* hit_slot_of_entry = (int32_t*)malloc(sizeof(int32_t) * (size_t)(top_k > 0 ? top_k : 1));
  uint8_t* slot_is_hit = (uint8_t*)malloc((size_t)S);
  uint8_t* entry_done = (uint8_t*)malloc((size_t)(top_k > 0 ? top_k : 1));
  if (!keys || !hit_slot_of_entry || !slot_is_hit || !entry_done) {
    free(keys); free(hit_slot_of_entry); free(slot_is_hit); free(entry_done);
    return OR_ENOMEM;
  }

  for (int32_t b = 0; b < batch; ++b) {
    int32_t* o = out + (int64_t)b * top_k;
    const int32_t* row = top_k_tokens + (int64_t)b * top_k;
    int32_t r = req_idx[b];

    /* Padding row ([P3] 7.1: padding batch rows output -1). */
    if (r < 0 || r >= R) {
      for (int32_t i = 0; i < top_k; ++i) o[i] = -1;
      if (r >= R) stats[ST_TRIP] += 1;
      continue;
    }

    int32_t* st = slot_tokens + (int64_t)r * S;
    int32_t* lru = lru_slots + (int64_t)r * S;
    int64_t n = seq_lens[b];
    if (n > max_seq_len) n = max_seq_len; /* memory-safety clamp */
    /* c = ++clock, computed without signed overflow. */
    int32_t c = (int32_t)((uint32_t)lru_clock[r] + 1u);
    lru_clock[r] = c;

    /* Fast path ([P2] "The flow of each decode step"): the whole sequence
     * already sits in the device buffer, slot = position, nothing moves. */
    if ((int64_t)seq_lens[b] <= (int64_t)S) {
      for (int32_t i = 0; i < top_k; ++i) {
        int32_t t = row[i];
        if (t < 0 || (int64_t)t >= n) { o[i] = -1; continue; }
        o[i] = r * S + t;
        st[t] = t;
        lru[t] = c;
        stats[ST_FAST] += 1;
      }
      continue;
    }

    /* LRU path. */
    for (int32_t i = 0; i < top_k; ++i) { entry_done[i] = 0; o[i] = -1; }

    /* Step 1: resident short-circuit ([P3] 7.2 phase 1; [P5] mixed
     * residency: resident tokens are read in place, no LRU, no copy). */
    for (int32_t i = 0; i < top_k; ++i) {
      int32_t t = row[i];
      if (t < 0 || (int64_t)t >= n) { entry_done[i] = 1; continue; }
      if (block_table != NULL && P > 0) {
        int32_t p = block_table[(int64_t)r * max_pages + t / P];
        if (p >= 0 && (int64_t)p < resident_pages) {
          o[i] = (int32_t)((int64_t)R * S + (int64_t)p * P + t % P);
          entry_done[i] = 1;
          stats[ST_RESIDENT] += 1;
        } else if (p >= 0) {
          stats[ST_TRIP] += 1; /* corrupt page id: not resident */
        }
      }
    }

    /* Step 2: hot hits ([P1] "Hot-row lookup and LRU": a hot row is reused
     * and its LRU entry refreshed).  The lowest slot holding t wins. */
    for (int32_t s = 0; s < S; ++s) slot_is_hit[s] = 0;
    for (int32_t i = 0; i < top_k; ++i) {
      hit_slot_of_entry[i] = -1;
      if (entry_done[i]) continue;
      int32_t t = row[i];
      for (int32_t s = 0; s < S; ++s) {
        if (st[s] == t) { hit_slot_of_entry[i] = s; break; }
      }
    }
    for (int32_t i = 0; i < top_k; ++i) {
      int32_t s = hit_slot_of_entry[i];
      if (s < 0) continue;
      o[i] = r * S + s;
      lru[s] = c;
      slot_is_hit[s] = 1;
      entry_done[i] = 1;
      stats[ST_HITS] += 1;
    }

    /* Step 3: victims ([P3] 7.2 phase 3; [P4] 2.4.3 stage 2: evict the
     * least recently used slots, empty space first). */
    int32_t nv = 0;
    for (int32_t s = 0; s < S; ++s) {
      if (slot_is_hit[s]) continue;
      keys[nv].occupied = st[s] >= 0 ? 1 : 0; /* -1 and below: empty */
      keys[nv].stamp = lru[s];
      keys[nv].slot = s;
      ++nv;
    }
    qsort(keys, (size_t)nv, sizeof(victim_key), cmp_victim);

    /* Step 4: the j-th miss in ascending top-k index takes the j-th victim;
     * its host row is copied into every layer's pool ([P3] 7.2 phase 3,
     * [P3] 7.4 follower layers, [P3] 7.2 out-of-range source zero-fill). */
    int32_t j = 0;
    for (int32_t i = 0; i < top_k; ++i) {
      if (entry_done[i]) continue;
      int32_t t = row[i];
      int32_t s = keys[j].slot; /* j < nv: misses <= top_k - hits <= nv */
      ++j;
      st[s] = t;
      lru[s] = c;
      o[i] = r * S + s;
      int64_t dst = (int64_t)r * S + s;
      int64_t h = host_cache_locs[(int64_t)r * max_seq_len + t];
      for (int32_t l = 0; l < L; ++l) {
        uint8_t* d = dev_pools[l] + dst * row_bytes;
        if (h >= 0 && h < host_pool_rows[l]) {
          memcpy(d, host_pools[l] + h * row_bytes, (size_t)row_bytes);
        } else {
          memset(d, 0, (size_t)row_bytes);
          stats[ST_TRIP] += 1;
        }
      }
      stats[ST_MISSES] += 1;
    }
  }

  free(keys);
  free(hit_slot_of_entry);
  free(slot_is_hit);
  free(entry_done);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Number formats of the 656-byte sparse-MLA row ([P3] section 9: 512 bytes  */
/* of fp8 NoPE latent, 16 bytes of scales, 128 bytes of bf16 RoPE).          */
/* ------------------------------------------------------------------------ */

/* OCP OFP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN; there
 * are no infinities. */
double oracle_e4m3_to_double(uint8_t v) {
  int sign = (v >> 7) & 1;
  int e = (v >> 3) & 15;
  int m = v & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_to_double(uint16_t v) {
  uint32_t bits = (uint32_t)v << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double row_scale(const uint8_t* row, int blk) {
  float f;
  memcpy(&f, row + 512 + 4 * blk, sizeof f); /* little-endian fp32 */
  return (double)f;
}

/*
 * oracle_sparse_mla_decode: attention of each (request, head) query over the
 * rows named by device_buffer_locs, as consumed by the sparse-MLA decode
 * backend ([P1] "Ownership": the attention backend consumes the device cache
 * and the physical row IDs; [P3] 7.3; row format [P3] section 9).
 *
 *   K_i = [ deq(latent_i) (512) ; rope_i (64) ],  V_i = deq(latent_i)
 *   deq(latent)[d] = e4m3(byte d) * scale[d / 128]
 *   z_i = softmax_scale * (q . K_i)   over the entries i with loc >= 0
 *   o   = sum_i softmax(z)_i * V_i    (o = 0 when no entry is valid)
 *
 * Everything is computed in float64.  q is bf16 [batch][heads][576];
 * out is float64 [batch][heads][512].  A location >= dev_pool_rows is
 * skipped like -1.  Each referenced row's K (and so V) is decoded to
 * float64 once per batch row, and each query once per head, before the
 * sums; the products and sums are the ones written above, in the same order.
 */
int oracle_sparse_mla_decode(int32_t batch, int32_t heads, int32_t top_k,
                             const uint16_t* q, const int32_t* locs,
                             const uint8_t* dev_pool, int64_t dev_pool_rows,
                             int32_t row_bytes, float softmax_scale,
                             double* out) {
  if (row_bytes < 656) return OR_EINVAL;
  const size_t nk = (size_t)(top_k > 0 ? top_k : 1);
  double* z = (double*)malloc(sizeof(double) * nk);
  double* kd = (double*)malloc(sizeof(double) * nk * 576); /* K_i; V_i = its first 512 */
  if (!z || !kd) {
    free(z);
    free(kd);
    return OR_ENOMEM;
  }
  const double scale = (double)softmax_scale;
  double qd[576];
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t* lb = locs + (int64_t)b * top_k;
    for (int32_t i = 0; i < top_k; ++i) {
      int32_t loc = lb[i];
      if (loc < 0 || (int64_t)loc >= dev_pool_rows) continue;
      const uint8_t* row = dev_pool + (int64_t)loc * row_bytes;
      double* ki = kd + (size_t)i * 576;
      for (int d = 0; d < 512; ++d)
        ki[d] = oracle_e4m3_to_double(row[d]) * row_scale(row, d / 128);
      for (int d = 0; d < 64; ++d) {
        uint16_t rv;
        memcpy(&rv, row + 528 + 2 * d, sizeof rv);
        ki[512 + d] = oracle_bf16_to_double(rv);
      }
    }
    for (int32_t h = 0; h < heads; ++h) {
      const uint16_t* qh = q + ((int64_t)b * heads + h) * 576;
      double* oh = out + ((int64_t)b * heads + h) * 512;
      for (int d = 0; d < 576; ++d) qd[d] = oracle_bf16_to_double(qh[d]);
      for (int d = 0; d < 512; ++d) oh[d] = 0.0;
      double zmax = -INFINITY;
      int any = 0;
      for (int32_t i = 0; i < top_k; ++i) {
        int32_t loc = lb[i];
        if (loc < 0 || (int64_t)loc >= dev_pool_rows) continue;
        const double* ki = kd + (size_t)i * 576;
        double acc = 0.0;
        for (int d = 0; d < 512; ++d) acc += qd[d] * ki[d];         /* latent part */
        for (int d = 0; d < 64; ++d) acc += qd[512 + d] * ki[512 + d]; /* rope part */
        z[i] = scale * acc;
        if (!any || z[i] > zmax) zmax = z[i];
        any = 1;
      }
      if (!any) continue;
      double denom = 0.0;
      for (int32_t i = 0; i < top_k; ++i) {
        int32_t loc = lb[i];
        if (loc < 0 || (int64_t)loc >= dev_pool_rows) continue;
        denom += exp(z[i] - zmax);
      }
      for (int32_t i = 0; i < top_k; ++i) {
        int32_t loc = lb[i];
        if (loc < 0 || (int64_t)loc >= dev_pool_rows) continue;
        const double* vi = kd + (size_t)i * 576;
        double p = exp(z[i] - zmax) / denom;
        for (int d = 0; d < 512; ++d) oh[d] += p * vi[d];
      }
    }
  }
  free(z);
  free(kd);
  return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Row mirror (eager backup) and hot-entry invalidation.                     */
/* ------------------------------------------------------------------------ */

/*
 * oracle_mirror_rows -- copy device rows back to host rows in layers
 * [layer_begin, layer_end): host_pool[l][host_rows[i]] = dev_pool[l][dev_rows[i]].
 *
 * Follows the per-step flow of [P2] (step 5: the row written by the
 * previous token is copied from the device back to the host pool) and the
 * row mirror of [P3] section 6 (rows written by the forward pass are
 * mirrored to their host rows, so that a later spill moves no data).
 * Readings: an entry whose device row is negative is padding (skipped, not
 * counted); a device row >= dev_pool_rows or a host row outside
 * [0, host_pool_rows[l]) skips that layer's copy and counts one tripwire.
 * With `validate`, two copied entries naming one host row are rejected.
 */
int oracle_mirror_rows(int32_t row_bytes, int32_t count, const int32_t* dev_rows,
                       const int64_t* host_rows, uint8_t* const* dev_pools,
                       int64_t dev_pool_rows, uint8_t* const* host_pools,
                       const int64_t* host_pool_rows, int32_t layer_begin, int32_t layer_end,
                       uint64_t* stats, int validate) {
  if (row_bytes <= 0 || count < 0 || layer_begin < 0 || layer_end < layer_begin) return OR_EINVAL;
  if (validate) {
    for (int32_t i = 0; i < count; ++i)
      for (int32_t j = i + 1; j < count; ++j)
        if (dev_rows[i] >= 0 && dev_rows[j] >= 0 && host_rows[i] == host_rows[j]) return OR_EINVAL;
  }
  for (int32_t l = layer_begin; l < layer_end; ++l) {
    for (int32_t i = 0; i < count; ++i) {
      const int32_t d = dev_rows[i];
      const int64_t h = host_rows[i];
      if (d < 0) continue;
      if ((int64_t)d >= dev_pool_rows || h < 0 || h >= host_pool_rows[l]) {
        stats[ST_TRIP] += 1;
        continue;
      }
      memcpy(host_pools[l] + h * row_bytes, dev_pools[l] + (int64_t)d * row_bytes,
             (size_t)row_bytes);
    }
  }
  return OR_OK;
}

/*
 * oracle_invalidate_tokens -- for each entry i, clear every hot slot of
 * request row req_rows[i] whose token lies in [tok_begin[i], tok_end[i]):
 * the slot becomes empty (token -1) with stamp 0, the state of a slot that
 * was never used.  Follows the precise clearing of rows rewritten by a
 * prefill in [P3] section 6 (hot-cache coherence); with the hot key being
 * the token position, "rewritten rows" are token ranges of a request.
 * Readings: req_rows[i] < 0 is padding; req_rows[i] >= R counts one
 * tripwire and clears nothing; an empty range clears nothing.
 */
int oracle_invalidate_tokens(int32_t R, int32_t S, int32_t count, const int32_t* req_rows,
                             const int32_t* tok_begin, const int32_t* tok_end,
                             int32_t* slot_tokens, int32_t* lru_slots, uint64_t* stats) {
  if (R <= 0 || S <= 0 || count < 0) return OR_EINVAL;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t r = req_rows[i];
    if (r < 0) continue;
    if (r >= R) {
      stats[ST_TRIP] += 1;
      continue;
    }
    for (int32_t s = 0; s < S; ++s) {
      const int32_t t = slot_tokens[(int64_t)r * S + s];
      if (t >= tok_begin[i] && t < tok_end[i]) {
        slot_tokens[(int64_t)r * S + s] = -1;
        lru_slots[(int64_t)r * S + s] = 0;
      }
    }
  }
  return OR_OK;
}

/*
 * oracle_invalidate_host_rows -- clear every hot slot (of every request row)
 * holding a token whose host row host_cache_locs[r][t] is one of the
 * `count` rows in `rows` (host rows that were reused for other content or
 * rewritten): token -1, stamp 0.  Follows [P3] section 6 (hot-cache
 * coherence: newly allocated host blocks are matched in a batch against the
 * hot entries, which must be cleared when their host rows are reused).
 * Tokens outside [0, max_seq_len) (empty or corrupted slots) are left alone.
 * With `validate`, `rows` must be sorted ascending (the form the kernel
 * searches).  Plain linear membership test.
 */
int oracle_invalidate_host_rows(int32_t R, int32_t S, int64_t max_seq_len, int32_t count,
                                const int64_t* rows, const int64_t* host_cache_locs,
                                int32_t* slot_tokens, int32_t* lru_slots, int validate) {
  if (R <= 0 || S <= 0 || count < 0 || max_seq_len <= 0) return OR_EINVAL;
  if (validate)
    for (int32_t i = 1; i < count; ++i)
      if (rows[i] < rows[i - 1]) return OR_EINVAL;
  for (int32_t r = 0; r < R; ++r) {
    for (int32_t s = 0; s < S; ++s) {
      const int32_t t = slot_tokens[(int64_t)r * S + s];
      if (t < 0 || (int64_t)t >= max_seq_len) continue;
      const int64_t h = host_cache_locs[(int64_t)r * max_seq_len + t];
      int found = 0;
      for (int32_t i = 0; i < count && !found; ++i) found = rows[i] == h;
      if (found) {
        slot_tokens[(int64_t)r * S + s] = -1;
        lru_slots[(int64_t)r * S + s] = 0;
      }
    }
  }
  return OR_OK;
}
