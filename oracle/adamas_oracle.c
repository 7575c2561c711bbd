/*
 * adamas_oracle.c -- plain, slow, CPU reference of the Adamas decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: only the pytest suites, the one-shot smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library; it is written from the method's description, not from the kernels.
 *
 * Sources (cited below by short name):
 *   [v2-abs]  "Adamas: Hadamard Sparse Attention for Efficient Long-Context
 *             Inference", arXiv 2510.18413 v2, abstract.
 *   [v1-abs]  the same paper, v1 abstract (as reproduced on chatpaper.ai and the
 *             mlsanity.com citation map).
 *   [blog]    "ADAMAS：稀疏注意力优化技术解析与应用实践" (jsqmd.com), with its
 *             section numbers (§2.1 Hadamard, §2.2 bucketing, §2.3 Manhattan
 *             distance, §3.1 compressed cache, §3.2 precision tuning, §6
 *             practice advice).
 *   [map]     the mlsanity.com citation-map page of the paper, "Builds on" list.
 *
 * Build: gcc -O2 -std=c99 -ffp-contract=off -fno-fast-math (no FMA contraction,
 * no reassociation: each float add/sub rounds once, in the order written).
 * Precision: the Hadamard transform runs in fp32 with a fixed butterfly order
 * (it decides the 2-bit codes, so its rounding is part of the definition);
 * attention runs in fp64.
 *
 * Every function takes host pointers.  Tensor layouts (row-major, contiguous):
 *   q      bf16 bits  [B][Hq][128]
 *   k, v   bf16 bits  [B][Hkv][cap][128]
 *   codes  u8         [B][Hkv][cap][32]   (packed 2-bit codes, planar layout)
 *   out    f32        [B][Hq][128]
 * Query head h reads KV head h / (Hq/Hkv) (contiguous GQA groups).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define HD 128         /* head dimension: the transform works on one head vector */
#define CODE_BYTES 32  /* 128 codes x 2 bits */
#define MAX_DIST 384   /* 128 coordinates x largest per-coordinate gap 3 */

/* bf16 -> fp32 is exact: the 16 stored bits are the top half of the fp32 word. */
float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/*
 * Unnormalised Walsh-Hadamard transform of one 128-vector, natural (Sylvester)
 * order: y[j] = sum_i (-1)^popcount(i & j) x[i].
 * [v2-abs]/[v1-abs]: the method Hadamard-transforms q and k; [blog §2.1]: the
 * transform is applied in O(n log n) by divide and conquer.
 * Reading: entries are +-1 (H H^T = 128 I), so q.k is kept up to the factor 128;
 * the stages run with half-width h = 1, 2, 4, ..., 64 in that order, and within a
 * stage each pair (a, b) = (x[j], x[j+h]) becomes (a + b, a - b), each sum
 * rounded once in fp32.  This order fixes the rounding of every output.
 */
void oracle_fwht128(const float* x, float* y) {
  float t[HD];
  memcpy(t, x, sizeof t);
  for (int h = 1; h < HD; h *= 2) {
    for (int base = 0; base < HD; base += 2 * h) {
      for (int j = base; j < base + h; ++j) {
        float a = t[j];
        float b = t[j + h];
        t[j] = a + b;
        t[j + h] = a - b;
      }
    }
  }
  memcpy(y, t, sizeof t);
}

/*
 * Dynamic 4-level bucketing of one transformed vector [blog §2.2]: the
 * thresholds are -t, 0, +t with t = 0.5 * max|y|, recomputed per vector (one
 * head vector is one 128-dimension group), and the code is the number of
 * thresholds the value is not below, using strict "<" tests:
 *   code 0 if y < -t, 1 if y < 0, 2 if y < t, else 3.
 * Consequences of the strict tests: y == -t -> 1, y == 0 or -0 -> 2, y == t -> 3;
 * an all-zero vector (t = 0) gives code 3 everywhere.  Inputs must be finite.
 */
void oracle_bucketize128(const float* y, uint8_t* codes) {
  float m = 0.0f;
  for (int i = 0; i < HD; ++i) {
    float a = fabsf(y[i]);
    if (a > m) m = a;
  }
  float t = 0.5f * m;
  for (int i = 0; i < HD; ++i) {
    uint8_t c;
    if (y[i] < -t)
      c = 0;
    else if (y[i] < 0.0f)
      c = 1;
    else if (y[i] < t)
      c = 2;
    else
      c = 3;
    codes[i] = c;
  }
}

/*
 * 2-bit packing of 128 codes into 32 bytes ([v2-abs]: 2-bit compression; the
 * pages give no byte layout -- [blog §3.1]'s shift example is garbled).
 * Reading (planar): bytes 0..15 hold the low bit of every code, bytes 16..31 the
 * high bit; within a plane, code i sits in byte i/8 at bit i%8.
 */
void oracle_pack128(const uint8_t* codes, uint8_t* out) {
  memset(out, 0, CODE_BYTES);
  for (int i = 0; i < HD; ++i) {
    uint8_t lo = codes[i] & 1u;
    uint8_t hi = (codes[i] >> 1) & 1u;
    out[i / 8] |= (uint8_t)(lo << (i % 8));
    out[16 + i / 8] |= (uint8_t)(hi << (i % 8));
  }
}

void oracle_unpack128(const uint8_t* in, uint8_t* codes) {
  for (int i = 0; i < HD; ++i) {
    uint8_t lo = (in[i / 8] >> (i % 8)) & 1u;
    uint8_t hi = (in[16 + i / 8] >> (i % 8)) & 1u;
    codes[i] = (uint8_t)(lo | (hi << 1));
  }
}

/* One bf16 head vector -> 32 code bytes: widen, transform, bucketize, pack. */
void oracle_encode_vector(const uint16_t* x_bf16, uint8_t* out32) {
  float x[HD], y[HD];
  uint8_t c[HD];
  for (int i = 0; i < HD; ++i) x[i] = oracle_bf16_to_f32(x_bf16[i]);
  oracle_fwht128(x, y);
  oracle_bucketize128(y, c);
  oracle_pack128(c, out32);
}

/*
 * Manhattan distance between two packed code vectors: sum over the 128
 * coordinates of |a_i - b_i|, computed on the integer codes (not on dequantised
 * values).  [v1-abs]: Manhattan-distance estimation drives the top-k;
 * [v2-abs]: a lightweight distance-based estimate.  Range 0..384.
 */
int oracle_distance(const uint8_t* a32, const uint8_t* b32) {
  uint8_t a[HD], b[HD];
  oracle_unpack128(a32, a);
  oracle_unpack128(b32, b);
  int d = 0;
  for (int i = 0; i < HD; ++i) d += abs((int)a[i] - (int)b[i]);
  return d;
}

typedef struct {
  uint16_t d;
  int32_t p;
} dist_pos;

static int cmp_dist_pos(const void* x, const void* y) {
  const dist_pos* a = (const dist_pos*)x;
  const dist_pos* b = (const dist_pos*)y;
  if (a->d != b->d) return a->d < b->d ? -1 : 1;
  if (a->p != b->p) return a->p < b->p ? -1 : 1;
  return 0;
}

static int cmp_i32(const void* x, const void* y) {
  int32_t a = *(const int32_t*)x, b = *(const int32_t*)y;
  return (a > b) - (a < b);
}

/*
 * Top-k under a token budget ([v2-abs]: top-k candidate selection over the
 * distance estimates; smallest distance = most similar code).
 * k_eff = min(budget, len).  Positions are ordered by (distance, position) --
 * the same order a stable sort by distance gives -- and the first k_eff are kept,
 * so among equal distances the lower position wins.  The kept positions are
 * written in ascending order; slots k_eff..budget-1 are set to -1.
 * Returns k_eff.
 */
int oracle_topk(const uint16_t* dist, int32_t len, int32_t budget, int32_t* sel) {
  int32_t k_eff = budget < len ? budget : len;
  dist_pos* v = (dist_pos*)malloc(sizeof(dist_pos) * (size_t)(len > 0 ? len : 1));
  for (int32_t p = 0; p < len; ++p) {
    v[p].d = dist[p];
    v[p].p = p;
  }
  qsort(v, (size_t)len, sizeof(dist_pos), cmp_dist_pos);
  for (int32_t i = 0; i < k_eff; ++i) sel[i] = v[i].p;
  qsort(sel, (size_t)k_eff, sizeof(int32_t), cmp_i32);
  for (int32_t i = k_eff; i < budget; ++i) sel[i] = -1;
  free(v);
  return k_eff;
}

typedef struct {
  uint8_t cls; /* 0: always kept, 1: preferred, 2: ranked by distance */
  uint16_t d;
  int32_t p;
} forced_dist_pos;

static int cmp_forced(const void* x, const void* y) {
  const forced_dist_pos* a = (const forced_dist_pos*)x;
  const forced_dist_pos* b = (const forced_dist_pos*)y;
  if (a->cls != b->cls) return a->cls < b->cls ? -1 : 1;
  if (a->cls == 2 && a->d != b->d) return a->d < b->d ? -1 : 1;
  if (a->p != b->p) return a->p < b->p ? -1 : 1;
  return 0;
}

/*
 * Top-k with forced positions.  [blog §3.2] and [blog §6]: special tokens (a
 * leading [CLS] is the example) should keep full attention, i.e. never be
 * dropped by the sparse selection; [map]: the paper builds on the
 * attention-sink work, whose first tokens are always attended.
 * Reading: force[p] = 2 marks a position that is always kept (a sink or a
 * recent-window position; the caller guarantees at most k_eff of them), 1 a
 * preferred position (a special token of the caller's mask), 0 an ordinary
 * one.  The k_eff = min(budget, len) kept positions are taken in this order:
 * the force-2 positions; then the force-1 positions, lower positions first;
 * then the ordinary positions by (distance, position) as in oracle_topk.  So
 * the rest of the budget after the always-kept positions goes to the special
 * tokens (the lowest ones if they do not all fit) and then to the closest
 * ordinary positions.  force == NULL: every position is ordinary (the result is
 * oracle_topk's).  Output as in oracle_topk.
 */
int oracle_topk_forced(const uint16_t* dist, const uint8_t* force, int32_t len, int32_t budget,
                       int32_t* sel) {
  int32_t k_eff = budget < len ? budget : len;
  forced_dist_pos* v = (forced_dist_pos*)malloc(sizeof(forced_dist_pos) * (size_t)(len > 0 ? len : 1));
  for (int32_t p = 0; p < len; ++p) {
    const int f = force ? force[p] : 0;
    v[p].cls = (uint8_t)(f >= 2 ? 0 : (f == 1 ? 1 : 2));
    v[p].d = dist[p];
    v[p].p = p;
  }
  qsort(v, (size_t)len, sizeof(forced_dist_pos), cmp_forced);
  for (int32_t i = 0; i < k_eff; ++i) sel[i] = v[i].p;
  qsort(sel, (size_t)k_eff, sizeof(int32_t), cmp_i32);
  for (int32_t i = k_eff; i < budget; ++i) sel[i] = -1;
  free(v);
  return k_eff;
}

/*
 * Exact softmax attention of one query over the listed rows of one KV head
 * ([v2-abs]: the selected positions gather the original K/V for sparse
 * attention).  s_p = scale * sum_i q_i K[p][i]; o = sum_p softmax(s)_p V[p].
 * Inputs are the original bf16 values; all arithmetic is fp64; out is rounded
 * to fp32 once at the end.  n == 0 (a sequence with no cached position) gives
 * the zero vector: the pages never attend over an empty set, and the empty sum
 * of weighted values is the reading taken (an idle slot of a batch).
 */
void oracle_attention_rows(const uint16_t* q, const uint16_t* kh, const uint16_t* vh,
                           const int32_t* pos, int32_t n, double scale, float* out) {
  if (n <= 0) {
    for (int i = 0; i < HD; ++i) out[i] = 0.0f;
    return;
  }
  double* s = (double*)malloc(sizeof(double) * (size_t)n);
  double qd[HD];
  for (int i = 0; i < HD; ++i) qd[i] = (double)oracle_bf16_to_f32(q[i]);
  double m = -INFINITY;
  for (int32_t r = 0; r < n; ++r) {
    const uint16_t* krow = kh + (size_t)pos[r] * HD;
    double dot = 0.0;
    for (int i = 0; i < HD; ++i) dot += qd[i] * (double)oracle_bf16_to_f32(krow[i]);
    s[r] = scale * dot;
    if (s[r] > m) m = s[r];
  }
  double l = 0.0;
  double o[HD];
  for (int i = 0; i < HD; ++i) o[i] = 0.0;
  for (int32_t r = 0; r < n; ++r) {
    double w = exp(s[r] - m);
    l += w;
    const uint16_t* vrow = vh + (size_t)pos[r] * HD;
    for (int i = 0; i < HD; ++i) o[i] += w * (double)oracle_bf16_to_f32(vrow[i]);
  }
  for (int i = 0; i < HD; ++i) out[i] = (float)(o[i] / l);
  free(s);
}

/* Argument checks shared by the batched entry points: 0 = ok, 1 = invalid. */
static int bad_dims(int32_t B, int32_t Hq, int32_t Hkv, int32_t cap) {
  return B < 1 || Hq < 1 || Hkv < 1 || cap < 1 || (Hq % Hkv) != 0;
}

/*
 * Key-code maintenance: for every batch entry b and KV head g, encode the keys
 * at positions [start[b], end[b]) (start may be NULL = 0).  The same routine
 * serves the prefill pass and the one-key append (start = len-1, end = len);
 * because thresholds are per vector, a key's code never depends on other keys.
 * threads > 1 encodes independent key rows in parallel (no change to any
 * arithmetic: each row is encoded by oracle_encode_vector alone).
 * Returns 0, or 1 on invalid arguments.
 */
int oracle_encode_keys(int32_t B, int32_t Hkv, int32_t cap, const uint16_t* k,
                       const int32_t* start, const int32_t* end, uint8_t* codes, int32_t threads) {
  if (bad_dims(B, Hkv, Hkv, cap)) return 1;
  for (int32_t b = 0; b < B; ++b) {
    int32_t s = start ? start[b] : 0;
    int32_t e = end[b];
    if (s < 0 || e > cap || s > e) return 1;
  }
  const int64_t rows = (int64_t)B * Hkv * cap;
  (void)threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1)
#endif
  for (int64_t row = 0; row < rows; ++row) {
    const int32_t b = (int32_t)(row / ((int64_t)Hkv * cap));
    const int32_t p = (int32_t)(row % cap);
    const int32_t s = start ? start[b] : 0;
    if (p >= s && p < end[b]) oracle_encode_vector(k + (size_t)row * HD, codes + (size_t)row * CODE_BYTES);
  }
  return 0;
}

/*
 * One decode step for every (b, query head h):
 *   1. encode q[b][h] (transform, bucketize, pack)  -> q_codes (optional output)
 *   2. dist[p] = Manhattan distance to codes[b][g][p] for p < kv_len[b]
 *      (optional output; entries at p >= kv_len[b] are left untouched)
 *   3. top-k with k_eff = min(budget, kv_len[b])       -> sel_idx (optional)
 *      with the forced positions of oracle_topk_forced: always kept are
 *      p < sink and p >= kv_len[b] - recent (sink + recent <= budget, so they
 *      fit); preferred are the positions whose bit p % 32 of
 *      mask[b * mask_words + p / 32] is set (mask may be NULL)
 *   4. exact fp64 softmax attention over the selected original K/V rows -> out
 * g = h / (Hq / Hkv).  0 <= kv_len[b] <= cap; a sequence with kv_len[b] = 0
 * selects nothing (sel_idx all -1) and gets the zero vector (see
 * oracle_attention_rows).  threads > 1 runs independent (b, h) pairs in parallel
 * (no change to any arithmetic).  Returns 0, or 1 on invalid arguments
 * (including sink < 0, recent < 0, sink + recent > budget, or a mask with
 * fewer than ceil(cap / 32) words per batch entry).
 */
int oracle_decode_step_forced(int32_t B, int32_t Hq, int32_t Hkv, int32_t cap,
                              const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const uint8_t* codes, const int32_t* kv_len, int32_t budget,
                              float scale, int32_t sink, int32_t recent, const uint32_t* mask,
                              int32_t mask_words, float* out, int32_t* sel_idx, uint16_t* dist,
                              uint8_t* q_codes, int32_t threads) {
  if (bad_dims(B, Hq, Hkv, cap) || budget < 1) return 1;
  if (sink < 0 || recent < 0 || (int64_t)sink + recent > budget) return 1;
  if (mask && (int64_t)mask_words * 32 < cap) return 1;
  for (int32_t b = 0; b < B; ++b)
    if (kv_len[b] < 0 || kv_len[b] > cap) return 1;
  const int32_t group = Hq / Hkv;
  const int32_t pairs = B * Hq;
  (void)threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1)
#endif
  for (int32_t bh = 0; bh < pairs; ++bh) {
    const int32_t b = bh / Hq, h = bh % Hq, g = h / group;
    const int32_t len = kv_len[b];
    const size_t nalloc = (size_t)(len > 0 ? len : 1);
    uint8_t qc[CODE_BYTES];
    oracle_encode_vector(q + (size_t)bh * HD, qc);
    if (q_codes) memcpy(q_codes + (size_t)bh * CODE_BYTES, qc, CODE_BYTES);
    const size_t kvbase = ((size_t)b * Hkv + g) * (size_t)cap;
    uint16_t* d = (uint16_t*)malloc(sizeof(uint16_t) * nalloc);
    for (int32_t p = 0; p < len; ++p)
      d[p] = (uint16_t)oracle_distance(qc, codes + (kvbase + (size_t)p) * CODE_BYTES);
    if (dist) memcpy(dist + (size_t)bh * cap, d, sizeof(uint16_t) * (size_t)len);
    uint8_t* f = (uint8_t*)malloc(nalloc);
    for (int32_t p = 0; p < len; ++p) {
      const int in_mask = mask ? (int)((mask[(size_t)b * mask_words + (size_t)(p / 32)] >> (p % 32)) & 1u) : 0;
      f[p] = (uint8_t)((p < sink || p >= len - recent) ? 2 : (in_mask ? 1 : 0));
    }
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)budget);
    int32_t k_eff = oracle_topk_forced(d, f, len, budget, sel);
    free(f);
    if (sel_idx) memcpy(sel_idx + (size_t)bh * budget, sel, sizeof(int32_t) * (size_t)budget);
    oracle_attention_rows(q + (size_t)bh * HD, k + kvbase * HD, v + kvbase * HD, sel, k_eff,
                          (double)scale, out + (size_t)bh * HD);
    free(sel);
    free(d);
  }
  return 0;
}

/* The decode step with no forced positions. */
int oracle_decode_step(int32_t B, int32_t Hq, int32_t Hkv, int32_t cap,
                       const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       const uint8_t* codes, const int32_t* kv_len, int32_t budget,
                       float scale, float* out, int32_t* sel_idx, uint16_t* dist,
                       uint8_t* q_codes, int32_t threads) {
  return oracle_decode_step_forced(B, Hq, Hkv, cap, q, k, v, codes, kv_len, budget, scale, 0, 0,
                                   NULL, 0, out, sel_idx, dist, q_codes, threads);
}

/*
 * Dense decode attention, the comparison baseline: the attention of step 4 over
 * every position p < kv_len[b] (the zero vector where kv_len[b] = 0).  Returns 0,
 * or 1 on invalid arguments.
 */
int oracle_dense_attention(int32_t B, int32_t Hq, int32_t Hkv, int32_t cap, const uint16_t* q,
                           const uint16_t* k, const uint16_t* v, const int32_t* kv_len,
                           float scale, float* out, int32_t threads) {
  if (bad_dims(B, Hq, Hkv, cap)) return 1;
  for (int32_t b = 0; b < B; ++b)
    if (kv_len[b] < 0 || kv_len[b] > cap) return 1;
  const int32_t group = Hq / Hkv;
  const int32_t pairs = B * Hq;
  (void)threads;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(threads > 0 ? threads : 1)
#endif
  for (int32_t bh = 0; bh < pairs; ++bh) {
    const int32_t b = bh / Hq, h = bh % Hq, g = h / group;
    const int32_t len = kv_len[b];
    const size_t kvbase = ((size_t)b * Hkv + g) * (size_t)cap;
    int32_t* all = (int32_t*)malloc(sizeof(int32_t) * (size_t)(len > 0 ? len : 1));
    for (int32_t p = 0; p < len; ++p) all[p] = p;
    oracle_attention_rows(q + (size_t)bh * HD, k + kvbase * HD, v + kvbase * HD, all, len,
                          (double)scale, out + (size_t)bh * HD);
    free(all);
  }
  return 0;
}
