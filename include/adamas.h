/*
 * adamas.h -- C ABI of the Adamas decode-step library (libadamas.so, gfx950).
 *
 * What the library computes (sources cited by page title and section):
 *   "Adamas: Hadamard Sparse Attention for Efficient Long-Context Inference"
 *   (arXiv 2510.18413), v1 and v2 abstracts: each query and key vector is
 *   Hadamard-transformed, bucketized and compressed to 2 bits; a distance
 *   estimate between the query's code and every key's code (Manhattan distance in
 *   v1) picks the top-k positions under a token budget; the original K/V rows at
 *   those positions are gathered and attended with exact softmax attention.
 *   "ADAMAS：稀疏注意力优化技术解析与应用实践" (jsqmd.com blog): section 2.1 (the
 *   transform, computed in O(n log n)), section 2.2 (dynamic thresholds
 *   -t, 0, +t with t = half the largest magnitude, strict "<" tests),
 *   section 2.3 (Manhattan distance on the integer codes), section 3.1 (key codes
 *   are kept in a cache that is updated as keys are appended).
 *
 * Fixed readings where the pages are silent or garbled:
 *   - head_dim is 128; the transform is the unnormalised Sylvester-Hadamard
 *     matrix in natural order, computed in fp32 by butterflies of half-width
 *     1, 2, 4, ..., 64 in that order (this fixes every rounding);
 *   - t is computed per head vector (one 128-dimension group);
 *   - codes are packed planar: bytes 0..15 hold the low bit of every code and
 *     bytes 16..31 the high bit, code i at bit i%8 of byte i/8 of each plane;
 *   - distance = sum over coordinates of |code_q - code_k|, in 0..384;
 *   - top-k keeps the min(budget, kv_len) positions with the smallest
 *     (distance, position) -- among equal distances the lower position wins;
 *   - attention uses the original bf16 q (not the transformed one) and a
 *     caller-supplied softmax scale (normally 1/sqrt(128));
 *   - query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Conventions for every call:
 *   - All tensor pointers are caller-owned DEVICE pointers to contiguous,
 *     row-major memory on the current HIP device.  bf16 tensors are passed as
 *     their raw 16-bit storage.  `stream` is a hipStream_t passed as void*
 *     (NULL = the null stream).
 *   - Calls only enqueue work on `stream` and return; results are ready when the
 *     stream reaches them.  No call allocates or frees device memory; scratch
 *     memory is the caller's `workspace` (adamas_decode_step_noalloc: a static
 *     array the library holds on each device).
 *   - Arguments the host can check are validated before any HIP call; on failure
 *     the call returns a status and enqueues nothing.  Values that live in
 *     device memory (kv_len, start, end) cannot be checked by the host: the
 *     kernels clamp them to [0, capacity], so no value makes a kernel read or
 *     write outside the buffers the dims describe, but results for values
 *     outside the stated preconditions are unspecified (kv_len = 0 is inside
 *     them: an empty sequence).
 *   - A failed launch returns ADAMAS_ERR_HIP.  The library keeps no mutable
 *     global state but the static scratch of adamas_decode_step_noalloc (the
 *     opt-in profiling setting below is per thread); calls on different streams
 *     with different workspaces may run concurrently.  Two calls that share a
 *     workspace (or two adamas_decode_step_noalloc calls on one GPU) must be
 *     ordered.
 */
#ifndef ADAMAS_H
#define ADAMAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ADAMAS_ABI_VERSION 1
#define ADAMAS_HEAD_DIM 128
#define ADAMAS_CODE_BYTES 32

typedef enum adamas_status {
  ADAMAS_OK = 0,
  ADAMAS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, budget < 1, ...          */
  ADAMAS_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. head_dim != 128)  */
  ADAMAS_ERR_WORKSPACE = 3,        /* workspace pointer NULL or smaller than required   */
  ADAMAS_ERR_HIP = 4               /* a HIP runtime call or kernel launch failed        */
} adamas_status;

/* Shapes shared by every call.  head_dim must be 128.  num_q_heads must be a
 * multiple of num_kv_heads, and the group size num_q_heads / num_kv_heads must be
 * 1, 2, 4 or 8.  capacity = allocated positions per (batch, kv head). */
typedef struct adamas_dims {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t capacity;
} adamas_dims;

/*
 * Key-code maintenance (prefill and append).  For every batch entry b and KV head
 * g, encode the keys at positions start[b] <= p < end[b]: transform, bucketize
 * and pack each key vector into 32 bytes.  Codes of other positions are not
 * touched.  Because thresholds are per vector, appending a key needs only that
 * key: after writing K[b][g][len-1], call with start = len-1, end = len.
 *   k      bf16 [batch][num_kv_heads][capacity][128]
 *   start  int32 [batch] device array, or NULL for all zeros
 *   end    int32 [batch] device array; precondition 0 <= start[b] <= end[b] <= capacity
 *   codes  uint8 [batch][num_kv_heads][capacity][32] (output)
 * num_q_heads is ignored here.  Errors: INVALID_ARGUMENT (null k/end/codes, bad
 * dims), UNSUPPORTED (head_dim != 128), HIP.
 */
adamas_status adamas_encode_keys(const adamas_dims* d, const void* k, const int32_t* start,
                                 const int32_t* end, uint8_t* codes, void* stream);

/* Bytes of workspace adamas_decode_step needs for these dims and budget (0 if
 * the arguments are invalid or the combination is unsupported).  Any alignment
 * of 256 bytes is sufficient.  (Its first 16.25 KB hold the single-launch
 * step's per-group generation counters and chunk flags; like the rest, they
 * need no initialisation.) */
size_t adamas_decode_workspace_size(const adamas_dims* d, int32_t budget);

/*
 * One Adamas decode step for every (b, query head h), with g = h / (Hq/Hkv):
 *   1. encode q[b][h] exactly as adamas_encode_keys encodes a key;
 *   2. dist[p] = sum_i |code_q[i] - code_k[b][g][p][i]| for p < kv_len[b];
 *   3. select the k_b = min(budget, kv_len[b]) positions with the smallest
 *      (dist, position);
 *   4. out[b][h] = sum_{p in S} softmax_p(scale * q.K[b][g][p]) V[b][g][p], exact
 *      softmax over the selected original bf16 rows, fp32 accumulation.
 * Arguments:
 *   q          bf16 [batch][num_q_heads][128]
 *   k, v       bf16 [batch][num_kv_heads][capacity][128] (the original cache)
 *   codes      uint8 [batch][num_kv_heads][capacity][32], valid for p < kv_len[b]
 *   kv_len     int32 [batch] device array; precondition 0 <= kv_len[b] <= capacity.
 *              kv_len[b] = 0 (an idle slot of the batch): nothing is selected
 *              (sel_idx row all -1) and out[b][h] = 0, the empty sum (the pages
 *              never attend over an empty set; this is the reading taken)
 *   budget     token budget k >= 1, any positive int32 (may exceed kv_len[b]: then every
 *              position is kept; past the capacity it plans like budget = capacity)
 *   scale      softmax scale
 *   out        fp32 [batch][num_q_heads][128] (output)
 *   sel_idx    optional (NULL = not written): int32 [batch][num_q_heads][budget];
 *              the selected positions in ascending order, then -1 padding
 *   dist       optional debug output (NULL = not written): uint16
 *              [batch][num_q_heads][capacity]; entries p >= kv_len[b] untouched
 *   q_codes    optional debug output (NULL = not written): uint8 [batch][num_q_heads][32]
 *   workspace  device scratch of at least adamas_decode_workspace_size(d, budget)
 *              bytes, 256-byte aligned; its contents need no initialisation and
 *              are meaningless after the call.
 * Codes, distances and sel_idx are deterministic integers; out is deterministic
 * for fixed inputs.  Errors: INVALID_ARGUMENT, UNSUPPORTED (also: a budget so
 * large at a large capacity that the per-head selection state exceeds one
 * block's on-chip memory -- the budget is supported whenever
 * adamas_decode_workspace_size returns nonzero), WORKSPACE, HIP.
 */
adamas_status adamas_decode_step(const adamas_dims* d, const void* q, const void* k, const void* v,
                                 const uint8_t* codes, const int32_t* kv_len, int32_t budget,
                                 float scale, float* out, int32_t* sel_idx, uint16_t* dist,
                                 uint8_t* q_codes, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): adamas_decode_step
 * with no workspace argument.  Its scratch is a static device array of
 * ADAMAS_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU it
 * runs on until the process ends; the first call on a device takes its
 * address (hipGetSymbolAddress), and no call allocates or frees memory.
 * Every call on one GPU shares that array, so calls that overlap on one GPU
 * (other streams, other threads) race and must be ordered by the caller.  The
 * kernels write every scratch word they read, so no clearing is needed.
 * Arguments, layouts, results and errors as adamas_decode_step, plus
 * UNSUPPORTED when adamas_decode_workspace_size(d, budget) exceeds
 * ADAMAS_NOALLOC_SCRATCH_BYTES (checked before any HIP call), and HIP when
 * the scratch address cannot be obtained.
 */
#define ADAMAS_NOALLOC_SCRATCH_BYTES (64 << 20)
adamas_status adamas_decode_step_noalloc(const adamas_dims* d, const void* q, const void* k, const void* v,
                                         const uint8_t* codes, const int32_t* kv_len, int32_t budget,
                                         float scale, float* out, int32_t* sel_idx, uint16_t* dist,
                                         uint8_t* q_codes, void* stream);

/*
 * The decode step with the key append folded in: encodes the key at position
 * kv_len[b]-1 of every (b, kv head) into `codes` -- exactly what
 * adamas_encode_keys(start = kv_len-1, end = kv_len) writes -- and then computes
 * what adamas_decode_step computes, with the new key competing like any other.
 * (The first kernel of the step encodes the key in the block that scans its
 * position, so the append costs no separate launch.)  Same arguments, layouts,
 * workspace size and errors as adamas_decode_step; `codes` is written at
 * positions kv_len[b]-1 only (nothing where kv_len[b] = 0).  Precondition:
 * K[b][g][kv_len[b]-1] holds the new key.
 */
adamas_status adamas_append_decode_step(const adamas_dims* d, const void* q, const void* k,
                                        const void* v, uint8_t* codes, const int32_t* kv_len,
                                        int32_t budget, float scale, float* out, int32_t* sel_idx,
                                        uint16_t* dist, uint8_t* q_codes, void* workspace,
                                        size_t workspace_bytes, void* stream);

/*
 * Positions a decode step always selects, whatever their distance.  The blog
 * (section 3.2, precision tuning; section 6, practice advice) keeps special
 * tokens such as a leading [CLS] at full attention; the paper builds on the
 * attention-sink work (the mlsanity.com citation map lists it), whose first
 * tokens are always attended; a window of the latest tokens is the usual
 * companion.  For a position p < kv_len[b]:
 *   always kept   p < sink, or p >= kv_len[b] - recent;
 *   preferred     (mask != NULL) bit p % 32 of mask[b * mask_words + p / 32] set.
 *   sink, recent  >= 0 with sink + recent <= budget (so the always-kept
 *                 positions fit the budget)
 *   mask          optional device bitmap uint32 [batch][mask_words], 4-byte
 *                 aligned; bits at p >= kv_len[b] are ignored
 *   mask_words    words per batch entry, >= ceil(capacity / 32) when mask != NULL
 */
typedef struct adamas_forced {
  int32_t sink;
  int32_t recent;
  const uint32_t* mask;
  int32_t mask_words;
} adamas_forced;

/*
 * The decode step with forced positions.  The k_b = min(budget, kv_len[b])
 * selected positions are, in this order of preference: every always-kept
 * position; the preferred positions, lower positions first; then the other
 * positions by (dist, position).  So the sinks and the window are always
 * attended, every special token of the mask is too whenever they fit the rest
 * of the budget (the lowest ones otherwise), and what remains goes to the
 * closest other positions.  With sink = recent = 0 and mask = NULL the result is
 * adamas_decode_step's (append = 0) or adamas_append_decode_step's (append = 1).
 * `dist` still reports the plain Manhattan distances.  Arguments, layouts,
 * workspace size and errors as adamas_append_decode_step (codes are written
 * only when append = 1), plus INVALID_ARGUMENT for a NULL `forced`, append not
 * 0 or 1, sink or recent < 0, sink + recent > budget, or a misaligned or too
 * narrow mask.
 */
adamas_status adamas_forced_decode_step(const adamas_dims* d, const adamas_forced* forced, int32_t append,
                                        const void* q, const void* k, const void* v, uint8_t* codes,
                                        const int32_t* kv_len, int32_t budget, float scale, float* out,
                                        int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* Bytes of workspace dense_decode_attention needs (0 if the dims are invalid). */
size_t dense_decode_workspace_size(const adamas_dims* d);

/*
 * Dense decode attention, the comparison baseline the pages measure Adamas
 * against: out[b][h] = softmax attention of q[b][h] over every position
 * p < kv_len[b] of KV head g = h / (Hq/Hkv) (0 where kv_len[b] = 0).  Same
 * layouts, preconditions and errors as adamas_decode_step.  One launch: each
 * block attends one chunk of positions and the last block of a (b, KV head)
 * group to finish merges the group's chunk partials.  The workspace needs no
 * initialisation (its per-group counters carry a tag of the call); calls that
 * share a workspace must not overlap in time (the same holds for every entry
 * point's workspace).
 */
adamas_status dense_decode_attention(const adamas_dims* d, const void* q, const void* k, const void* v,
                                     const int32_t* kv_len, float scale, float* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Paged caches.  The pages are silent on cache layout; serving systems keep K/V
 * in fixed-size pages handed out from pools (the paper builds on FlashInfer, a
 * paged-KV attention engine, per the mlsanity.com citation map), and the key
 * codes of the blog's section 3.1 cache can share the same pages.  Position p of
 * sequence b lives on page block_table[b * max_pages + p / page_size] at slot
 * p % page_size:
 *   K, V pools    bf16  [num_pages][num_kv_heads][page_size][128]
 *   codes pool    uint8 [num_pages][num_kv_heads][page_size][32]
 *   block_table   int32 [batch][max_pages], device; page ids in [0, num_pages)
 *                 (a precondition like kv_len: ids outside are clamped, never
 *                 dereferenced out of the pools)
 *   page_size     a power of two (1 .. 2^20)
 *   max_pages     max_pages * page_size >= capacity (the dims' capacity is the
 *                 longest a sequence may grow)
 * Pages may be shared between sequences only where their contents are equal
 * (a common prefix); an append writes the page of position kv_len[b]-1.
 */
typedef struct adamas_pages {
  const int32_t* block_table;
  int32_t max_pages;
  int32_t page_size;
  int32_t num_pages;
} adamas_pages;

/* adamas_encode_keys on paged pools: encodes positions [start[b], end[b]) of
 * every sequence from k_pool into codes_pool.  Errors as adamas_encode_keys,
 * plus INVALID_ARGUMENT for a NULL or inconsistent `pages`. */
adamas_status adamas_paged_encode_keys(const adamas_dims* d, const adamas_pages* pages, const void* k_pool,
                                       const int32_t* start, const int32_t* end, uint8_t* codes_pool,
                                       void* stream);

/*
 * adamas_encode_keys (and its paged form) for a caller that knows, on the host,
 * a bound on how many positions each range holds -- an append of one key per
 * step (max_rows = 1), a chunked prefill.  The ranges stay in device memory, so
 * without the bound the launch is sized for the whole capacity; with it, for
 * max_rows positions per (b, kv head).  Same operation and outputs (the blog
 * "ADAMAS：稀疏注意力优化技术解析与应用实践", section 3.1: key codes maintained
 * per appended key).
 *   max_rows  > 0; intended: >= end[b] - start[b] for every b.  It sizes the grid
 *             only: every block walks its positions with a stride, so a bound that
 *             is too small encodes every position all the same, only more slowly.
 * Errors: as adamas_encode_keys / adamas_paged_encode_keys, plus INVALID_ARGUMENT
 * for max_rows < 1.
 */
adamas_status adamas_encode_keys_bounded(const adamas_dims* d, const void* k, const int32_t* start,
                                         const int32_t* end, int32_t max_rows, uint8_t* codes, void* stream);
adamas_status adamas_paged_encode_keys_bounded(const adamas_dims* d, const adamas_pages* pages,
                                               const void* k_pool, const int32_t* start, const int32_t* end,
                                               int32_t max_rows, uint8_t* codes_pool, void* stream);

/* The decode step on paged pools: what adamas_forced_decode_step computes
 * (forced may be NULL: no forced positions; append 0 or 1), reading K, V and
 * codes through the block table.  dist and sel_idx stay indexed by position.
 * Workspace: adamas_decode_workspace_size(d, budget).  Errors as
 * adamas_forced_decode_step, plus INVALID_ARGUMENT for a NULL or inconsistent
 * `pages`. */
adamas_status adamas_paged_decode_step(const adamas_dims* d, const adamas_pages* pages, const adamas_forced* forced,
                                       int32_t append, const void* q, const void* k_pool, const void* v_pool,
                                       uint8_t* codes_pool, const int32_t* kv_len, int32_t budget, float scale,
                                       float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* dense_decode_attention on paged pools (workspace: dense_decode_workspace_size). */
adamas_status dense_paged_decode_attention(const adamas_dims* d, const adamas_pages* pages, const void* q,
                                           const void* k_pool, const void* v_pool, const int32_t* kv_len,
                                           float scale, float* out, void* workspace, size_t workspace_bytes,
                                           void* stream);

/*
 * Profiling aid, not needed for correct use.  Enables (n_events > 0) or disables
 * (events == NULL or n_events == 0) per-kernel timing for calls made later on the
 * CALLING THREAD: launch i of a call (counting from 0) is bracketed by the HIP
 * events events[2*i] (start) and events[2*i+1] (stop), recorded on the call's
 * stream by the kernel dispatch itself, for every i with 2*i+1 < n_events.
 * Launch order: adamas_encode_keys, adamas_paged_encode_keys and their _bounded
 * forms -> 0 encode;
 * adamas_decode_step, adamas_append_decode_step, adamas_forced_decode_step and
 * adamas_paged_decode_step -> 0 scan, 1 select+attend (or 0 the single-launch
 * step, see adamas_decode_launch_mode); dense_decode_attention
 * and dense_paged_decode_attention -> 0 attend (and merge).  While timing is on, a call waits (on the host) for each
 * of its kernels before launching the next, so that every event pair brackets
 * one kernel and not the dispatch gap after the previous one.
 *   events    array of hipEvent_t handles (as void*) created by the caller with
 *             timing enabled; the array is copied, the events stay the caller's
 *   n_events  at most 16
 * Errors: INVALID_ARGUMENT if n_events < 0 or > 16, or events is NULL with
 * n_events > 0.  The setting is thread-local; it changes no result.
 */
adamas_status adamas_profile_events(void* const* events, int32_t n_events);

/*
 * How later decode steps of the CALLING THREAD are launched (a tuning and
 * testing aid; results are the same either way):
 *   mode 0 (default)  two kernels: scan, then select + attend;
 *   mode 1            one kernel per step where the shape allows it -- at most
 *                     64 (batch, kv head) groups, at most 32 chunks of the
 *                     scan per group, a chunk's block for every (query head,
 *                     split) of its group, and every block of the grid
 *                     resident on the device at once; the chunks' records are
 *                     written through to memory and handed to the selecting
 *                     blocks by per-chunk flags inside the kernel.  (On MI355X
 *                     this hand-off costs more than the kernel boundary it
 *                     replaces, so it is not the default.)
 * Applies to adamas_decode_step, adamas_append_decode_step,
 * adamas_forced_decode_step, adamas_paged_decode_step and
 * adamas_decode_step_noalloc.  With one kernel, adamas_profile_events slot 0
 * brackets it and slot 1 is not recorded.  Errors: INVALID_ARGUMENT for a mode
 * other than 0 or 1.
 */
adamas_status adamas_decode_launch_mode(int32_t mode);

/* Kernels launched by the calling thread's last decode step call (1 or 2; 0
 * if it launched none). */
int32_t adamas_last_launch_count(void);

/* Static, NUL-terminated description of a status code. */
const char* adamas_status_string(adamas_status s);

/* ADAMAS_ABI_VERSION of the built library. */
int32_t adamas_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ADAMAS_H */
