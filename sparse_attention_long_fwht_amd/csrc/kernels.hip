// kernels.hip -- key encode and the dense decode-attention baseline (gfx950).
//
// Sources (by page title and section):
//   "Adamas: Hadamard Sparse Attention for Efficient Long-Context Inference",
//   v1/v2 abstracts: keys are Hadamard-transformed, bucketized and compressed to
//   2-bit codes; Adamas is measured against full (dense) attention.
//   "ADAMAS：稀疏注意力优化技术解析与应用实践" blog: section 2.2 (thresholds),
//   section 3.1 (key codes kept in a cache updated per appended key).
//
// encode_keys_kernel   transform + bucketize + pack every key in [start, end)
//                      (prefill and append), four lanes per key vector
// dense_attend_kernel  per (b, kv head, chunk): exact softmax attention of the
//                      group's R queries over every cached position of the chunk,
//                      one (m, l, o) partial per head; the block that finds all
//                      of its group's partials in place merges them into out
// (The sparse decode step itself lives in decode.hip.)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "plan.h"

namespace adamas {

// --------------------------------------------------------------------------
// Key encode
// --------------------------------------------------------------------------

// grid (nblk, B*Hkv), 256 threads = 64 vectors per pass (a quad per vector).
// (every argument a block needs before its first loads is a leading scalar,
// preloaded into SGPRs at wave launch; the layout struct follows)
template <bool kPaged>
__global__ __launch_bounds__(256) void encode_keys_kernel(const uint16_t* __restrict__ k,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ end,
                                                          uint8_t* __restrict__ codes, int Hkv, uint32_t hkv_m,
                                                          int cap, KvLayout kv0) {
  KvLayout kv = kv0;
  kv.Hkv = Hkv;
  kv.hkv_m = hkv_m;
  kv.cap = cap;
  const int bg = blockIdx.y;
  const int b = div_by(bg, kv.Hkv, kv.hkv_m);
  const int g = bg - b * kv.Hkv;
  // (0 <= start <= end <= capacity is a precondition; clamped all the same)
  const int s = max(start ? start[b] : 0, 0);
  const int e = min(end[b], kv.cap);
  const int quarter = threadIdx.x & 3;
  const int slot = threadIdx.x >> 2;  // 0..63
  // The loop bound depends only on blockIdx, so every quad runs every pass.
  for (int p0 = s + (int)blockIdx.x * 64; p0 < e; p0 += (int)gridDim.x * 64) {
    const int p = p0 + slot;
    const bool valid = p < e;
    const int pl = valid ? p : e - 1;  // clamped rows keep the loads in bounds
    const size_t row = kPaged ? kv_row<true>(kv, b, g, pl) : (size_t)bg * (size_t)kv.cap + (size_t)pl;
    const uint4* src = reinterpret_cast<const uint4*>(k + row * kHeadDim + quarter * 32);
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = src[i];
    float x[32];
    widen32(w, x);
    uint32_t lo, hi;
    encode_quad(x, quarter, lo, hi);
    if (valid) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * kCodeBytes);  // (valid: row of p)
      dst[quarter] = lo;
      dst[4 + quarter] = hi;
    }
  }
}

// --------------------------------------------------------------------------
// Dense decode attention
// --------------------------------------------------------------------------

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  float* ws_part;       // [B][Hq][nch][kPartFloats]
  unsigned long long* ws_gen;  // [B][Hkv]: the group's generation, advanced once per call
  float* out;           // [B][Hq][128]
  float qscale;         // softmax scale * log2(e)
  int Hq, Hkv, cap, chunk, nch;
  KvLayout kv;
};

// Merge the per-chunk partials (m, l, o[128]) of R heads into out.  `part`
// points at head 0's partials; head r's are r * nch chunks further.  Runs with
// all kThreads threads of the block.  Up to kBatch chunks its reads of the
// partials are one round of loads: every load is issued before any is used
// (indices past the last chunk read the last chunk again).
template <int R, int kThreads>
__device__ __forceinline__ void combine_group(const float* __restrict__ part, int nch, int nch_b,
                                              float* __restrict__ out, float (*s_w)[kMaxChunks], float* s_L,
                                              unsigned long long* genp, unsigned long long gen) {
  // (the partials were written through by other blocks of this kernel: read
  // them coherently)
  auto ld = [](const float* p) {
    return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
  };
  const int tid = threadIdx.x;
  // 0. the election: of the blocks that found the group complete, the one
  // whose compare-and-swap advances the generation merges (no retry: a failed
  // swap means another block won).  Issued before the loads of step 1, its
  // round trip overlaps theirs.
  __shared__ int s_won;
  unsigned long long seen = ~gen;
  if (tid == 0) {
    unsigned long long expected = gen;
    __hip_atomic_compare_exchange_strong(genp, &expected, gen + 1, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    seen = expected;  // the word's value before the swap (gen iff it succeeded)
  }
  // 1. m and l of every (head, chunk)
  constexpr int kIt = (R * kMaxChunks + kThreads - 1) / kThreads;
  float mv[kIt], lv[kIt];
#pragma unroll
  for (int k = 0; k < kIt; ++k) {
    const int i = min(tid + k * kThreads, R * kMaxChunks - 1);
    const int r = i / kMaxChunks, c = i - r * kMaxChunks;
    const float* pc = part + ((size_t)r * nch + min(c, nch_b - 1)) * kPartFloats;
    mv[k] = ld(pc);
    lv[k] = ld(pc + 1);
  }
  // The o values of the first kBatch chunks (step 3) are requested now too:
  // their loads need no weight, so they share this round trip.
  constexpr int kPer = (R * kHeadDim + kThreads - 1) / kThreads;
  constexpr int kBatch = 64 / kPer;
  const float* pr[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = min(tid + k * kThreads, R * kHeadDim - 1);
    pr[k] = part + (size_t)(i / kHeadDim) * nch * kPartFloats + 4 + (i % kHeadDim);
  }
  float v[kPer][kBatch];
  auto load_batch = [&](int c0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k)
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[k][u] = ld(pr[k] + (size_t)min(c0 + u, nch_b - 1) * kPartFloats);
  };
  load_batch(0);
  // (the empty asm takes `seen` as an operand after the loads above are
  // issued, so the wait for the swap's result is not placed before them)
  asm volatile("" : "+v"(seen) : : "memory");
  if (tid == 0) s_won = seen == gen;
#pragma unroll
  for (int k = 0; k < kIt; ++k) {
    const int i = tid + k * kThreads;
    if (kIt * kThreads != R * kMaxChunks && i >= R * kMaxChunks) continue;
    const int r = i / kMaxChunks, c = i - r * kMaxChunks;
    s_w[r][c] = c < nch_b ? mv[k] : -INFINITY;
    if (c < nch_b) s_L[R + r * kMaxChunks + c] = lv[k];  // scratch: l values after the R totals
  }
  __syncthreads();
  if (!s_won) return;
  // 2. per head: M = max m, weights 2^(m - M), L = sum weight * l
  for (int r = wave_id(); r < R; r += kThreads / 64) {
    const int lane = lane_id();
    const float m0 = s_w[r][lane], m1 = s_w[r][lane + 64];
    const float M = wave_max(fmaxf(m0, m1));
    const float w0 = m0 == -INFINITY ? 0.f : exp2f(m0 - M);
    const float w1 = m1 == -INFINITY ? 0.f : exp2f(m1 - M);
    const float l0 = lane < nch_b ? s_L[R + r * kMaxChunks + lane] : 0.f;
    const float l1 = lane + 64 < nch_b ? s_L[R + r * kMaxChunks + lane + 64] : 0.f;
    const float L = wave_sum(w0 * l0 + w1 * l1);
    s_w[r][lane] = w0;
    s_w[r][lane + 64] = w1;
    if (lane == 0) s_L[r] = L;
  }
  __syncthreads();
  // 3. out[r][d] = sum_c w_c o_c[d] / L over the thread's kPer outputs, the
  // o values of kBatch chunks of each at a time (64 loads per thread; the
  // first batch was requested with step 1).  The weights of chunks past
  // nch_b are 0 (step 2) and their clamped loads read a finite partial, so
  // every term is added unconditionally; the weights come from LDS 16 bytes
  // at a time.  (Guarding each term and reading its weight alone made the
  // terms a chain of LDS round trips.)
  float O[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) O[k] = 0.f;
  for (int c0 = 0; c0 < nch_b; c0 += kBatch) {
    if (c0 > 0) load_batch(c0);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int r = min(tid + k * kThreads, R * kHeadDim - 1) / kHeadDim;
      const float4* wr = reinterpret_cast<const float4*>(&s_w[r][c0]);
#pragma unroll
      for (int u4 = 0; u4 < kBatch / 4; ++u4) {
        const float4 wq = wr[u4];
        O[k] = __builtin_fmaf(wq.x, v[k][4 * u4], O[k]);
        O[k] = __builtin_fmaf(wq.y, v[k][4 * u4 + 1], O[k]);
        O[k] = __builtin_fmaf(wq.z, v[k][4 * u4 + 2], O[k]);
        O[k] = __builtin_fmaf(wq.w, v[k][4 * u4 + 3], O[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int i = tid + k * kThreads;
    if (R * kHeadDim % kThreads == 0 || i < R * kHeadDim) out[i] = O[k] / s_L[i / kHeadDim];
  }
}

// lane (16 k + h)'s value for every lane 16 k + j of its 16-lane row (DPP
// row_newbcast)
template <int H>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + H, 0xF, 0xF, false));
}

constexpr int kDenseWaves = 4;  // waves per dense block; each streams its own 16-row tiles

// Exact softmax attention of the group's R queries over positions
// [p0, p0 + nrows) of one KV head, written as one partial (m, l, o[128]) per
// head: m = running max of the scaled log2 scores, l = sum 2^(s - m),
// o = sum 2^(s - m) V.  Wave w takes the 16-row tiles w, w + 4, ... and keeps
// its own online softmax; the K/V rows of its next two tiles are loaded while
// it computes the current one, and no barrier is taken until the four waves'
// partials are merged at the end.
//   q . K^T: MFMA 16x16x32 bf16, the tile's rows as the A operand and the R
//            heads as columns 0..R-1 of B: lane (col, kg) gets the scores of
//            rows 4 kg + i (i = 0..3) for head col;
//   softmax: per head, over those lanes (lane swaps across the 16-lane rows);
//   P . V:   lane (col, kg) accumulates dims 8 col .. 8 col + 7 of every head
//            over rows 4 kg + i, taking head h's probabilities from lane
//            (h, kg) of its row (DPP row broadcast); the four k-groups are
//            summed once, at the end.
template <int R, bool kPaged>
__device__ __forceinline__ void attend_rows(const AttendArgs& a, int b, int g, int c, int p0, int nrows) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int col = lane & 15;
  const int kg = lane >> 4;
  __shared__ float s_m[kDenseWaves][R], s_l[kDenseWaves][R];
  __shared__ float s_o[kDenseWaves][R][kHeadDim];

  uint4 qf[4];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)(g * R + (col < R ? col : 0))) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = col < R ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * kg) : make_uint4(0, 0, 0, 0);
  }
  // K and V rows of position p: Kg + kvoff(p), Vg + kvoff(p)
  const size_t kv_base = kPaged ? (size_t)0 : ((size_t)b * a.Hkv + g) * (size_t)a.cap * kHeadDim;
  const uint16_t* Kg = a.k + kv_base;
  const uint16_t* Vg = a.v + kv_base;
  auto kvoff = [&](int p) -> size_t {
    if constexpr (kPaged) return kv_row<true>(a.kv, b, g, p) * kHeadDim;
    else return (size_t)p * kHeadDim;
  };
  // The wave's rows of tile t.  Rows past nrows read the tile's first row, and
  // a tile past the last one (a request ahead of the end) reads row p0: in
  // bounds, finite, and on the tile's own page.  Pages of 16 positions or more
  // hold a whole tile (p0 is a multiple of 16), so the tile takes one
  // block-table entry, read through the scalar unit: its wait is then not one
  // on the vector loads still in flight for the tiles ahead.
  auto gather = [&](int t, uint4 (&ka)[4], uint4 (&vv)[4]) {
    const int r0 = 16 * t < nrows ? 16 * t : 0;
    const int ia = 16 * t + col < nrows ? 16 * t + col : r0;
    int iv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) iv[i] = 16 * t + 4 * kg + i < nrows ? 16 * t + 4 * kg + i : r0;
    size_t ok, ov[4];
    if (kPaged && a.kv.page_log2 >= 4) {
      const int mask = (1 << a.kv.page_log2) - 1;
      const int32_t* entry = a.kv.table + (size_t)b * a.kv.max_pages + ((p0 + r0) >> a.kv.page_log2);
      const int page = min(max(*reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(
                                   reinterpret_cast<uintptr_t>(entry)), 0), a.kv.num_pages - 1);
      const size_t base = (((size_t)page * a.Hkv + g) << a.kv.page_log2);
      ok = (base + ((p0 + ia) & mask)) * kHeadDim;
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = (base + ((p0 + iv[i]) & mask)) * kHeadDim;
    } else {
      ok = kvoff(p0 + ia);
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = kvoff(p0 + iv[i]);
    }
    const uint16_t* kr = Kg + ok + 8 * kg;
#pragma unroll
    for (int s = 0; s < 4; ++s) ka[s] = *reinterpret_cast<const uint4*>(kr + 32 * s);
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = *reinterpret_cast<const uint4*>(Vg + ov[i] + 8 * col);
  };
  float m_run = -INFINITY, l_run = 0.f;  // head col's running max and sum (lanes col < R)
  float o[R][8];
#pragma unroll
  for (int h = 0; h < R; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[h][j] = 0.f;
  const int ntiles = (nrows + 15) >> 4;
  // one tile: scores, online softmax update and P . V from its K rows ka and
  // V rows vv
  auto tile = [&](int t, const uint4 (&ka)[4], const uint4 (&vv)[4]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_16x16x32_bf16(ka[s], qf[s], acc);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = 16 * t + 4 * kg + i < nrows ? acc[i] * a.qscale : -INFINITY;
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __uint_as_float(xor16_u32(__float_as_uint(mx))));
    mx = fmaxf(mx, __uint_as_float(xor32_u32(__float_as_uint(mx))));
    const float m_new = fmaxf(m_run, mx);  // (finite: every tile has a valid row)
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run is -inf
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - m_new);
    float ls = (pr[0] + pr[1]) + (pr[2] + pr[3]);
    ls += __uint_as_float(xor16_u32(__float_as_uint(ls)));
    ls += __uint_as_float(xor32_u32(__float_as_uint(ls)));
    l_run = __builtin_fmaf(l_run, corr, ls);
    m_run = m_new;
    float vf[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t vw[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[i][2 * j] = bf16_lo(vw[j]);
        vf[i][2 * j + 1] = bf16_hi(vw[j]);
      }
    }
    auto pv = [&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float ch = row_bcast<h>(corr);
      float ph[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ph[i] = row_bcast<h>(pr[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float x = o[h][j] * ch;
#pragma unroll
        for (int i = 0; i < 4; ++i) x = __builtin_fmaf(ph[i], vf[i][j], x);
        o[h][j] = x;
      }
    };
    pv(std::integral_constant<int, 0>{});
    if constexpr (R > 1) pv(std::integral_constant<int, 1>{});
    if constexpr (R > 2) {
      pv(std::integral_constant<int, 2>{});
      pv(std::integral_constant<int, 3>{});
    }
    if constexpr (R > 4) {
      pv(std::integral_constant<int, 4>{});
      pv(std::integral_constant<int, 5>{});
      pv(std::integral_constant<int, 6>{});
      pv(std::integral_constant<int, 7>{});
    }
  };
  // Three register sets take the wave's tiles in turn, so that tiles t + 4
  // and t + 8 are in flight while tile t is computed.  (Rotating one set into
  // another instead makes the compiler copy registers, and a copy waits for
  // its load: the tile ahead would then have to land before the current one
  // is computed.)  The requests are issued unconditionally -- past the last
  // tile gather reads row p0 -- and every request is fenced on both sides
  // (`issue`): an empty asm with a memory clobber keeps the compiler from
  // sinking the loads down to the tile that uses them, and a scheduling
  // barrier keeps it from hoisting a later tile's arithmetic above them or
  // from interleaving two tiles' loads (the wait before a tile counts the
  // loads issued after it, and one count serves every iteration); neither
  // emits an instruction or a wait.  The loop takes whole triples and has one
  // exit: an exit from its middle would reach the loop's head, for the
  // compiler, with the third set's loads still pending, and the head would
  // wait for them.  The last one or two tiles follow it.
  auto issue = [&](int t, uint4 (&ka)[4], uint4 (&vv)[4]) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    gather(t, ka, vv);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  const int nt = ntiles > w ? (ntiles - w + kDenseWaves - 1) / kDenseWaves : 0;  // the wave's tiles
  uint4 ka[4], va[4], kb[4], vb[4], kc[4], vc[4];
  issue(w, ka, va);
  issue(w + kDenseWaves, kb, vb);
  int t = w;
#pragma unroll 1
  for (int n = nt; n >= 3; n -= 3, t += 3 * kDenseWaves) {
    issue(t + 2 * kDenseWaves, kc, vc);
    tile(t, ka, va);
    issue(t + 3 * kDenseWaves, ka, va);
    tile(t + kDenseWaves, kb, vb);
    issue(t + 4 * kDenseWaves, kb, vb);
    tile(t + 2 * kDenseWaves, kc, vc);
  }
  const int left = nt % 3;
  if (left >= 1) tile(t, ka, va);
  if (left == 2) tile(t + kDenseWaves, kb, vb);
  // the wave's partials: o summed over its four k-groups; m and l of head h
  // sit in lane h
#pragma unroll
  for (int h = 0; h < R; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = o[h][j];
      v += __uint_as_float(xor16_u32(__float_as_uint(v)));
      v += __uint_as_float(xor32_u32(__float_as_uint(v)));
      o[h][j] = v;
    }
  if (kg == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) s_o[w][h][8 * col + j] = o[h][j];
  }
  if (lane < R) {
    s_m[w][lane] = m_run;  // -inf for a wave without rows
    s_l[w][lane] = l_run;
  }
  __syncthreads();
  for (int i = tid; i < R * kHeadDim; i += kDenseWaves * 64) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kDenseWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDenseWaves; ++ww) {
      const float mw = s_m[ww][h];
      const float wt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L = __builtin_fmaf(s_l[ww][h], wt, L);
      O = __builtin_fmaf(s_o[ww][h][d], wt, O);
    }
    // written through, for the group's merging block in this same kernel
    uint32_t* pc = reinterpret_cast<uint32_t*>(a.ws_part) +
                   (((size_t)b * a.Hq + (size_t)(g * R + h)) * a.nch + c) * kPartFloats;
    if (d == 0) {
      __hip_atomic_store(pc, __float_as_uint(M), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pc + 1, __float_as_uint(L), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(pc + 4 + d, __float_as_uint(O), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The tag chunk c of a group writes beside its partial in a call whose
// generation is gen: a 64-bit hash (a splitmix64 finalizer), so that no partial
// left by another call, and no other content of the workspace, matches it.
__device__ __forceinline__ unsigned long long chunk_tag(unsigned long long gen, int c) {
  unsigned long long z = gen * 0x100000001B3ull + (unsigned long long)c + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Dense decode attention: block (c, b*Hkv + g) attends the group's R queries
// over positions [c*chunk, min((c+1)*chunk, kv_len[b])) and writes one partial
// per head; a block that finds every chunk's partial of its group in place
// merges them into out.  No block waits for another:
//   - every block reads the group's generation word when it starts;
//   - it writes its partial through to the point of coherence, then a tag of
//     (generation, chunk) in the pad words of its head-0 partial;
//   - it then reads every chunk's tag; if all match, the group is complete
//     (a tag is written only after its partial), and the block tries to
//     advance the generation with a compare-and-swap: the one block that
//     succeeds merges.
// Of blocks finishing together at least one sees all tags (each reads only
// after its own tag has reached the point of coherence), so exactly one
// merges.  The next call sees the new generation, so tags left by this one
// never match; arbitrary workspace content matches no hash, so the workspace
// needs no initialisation.
template <int R, bool kPaged>
// (the values a block needs before its first loads come first, as scalar
// arguments that gfx950 preloads into SGPRs at wave launch; the library is
// built with -amdgpu-kernarg-preload-count=16)
__global__ __launch_bounds__(kDenseWaves * 64) void dense_attend_kernel(const uint16_t* q, const uint16_t* k,
                                                                      const uint16_t* v, const int32_t* kv_len,
                                                                      int Hkv, uint32_t hkv_m, int cap, int chunk,
                                                                      AttendArgs a0) {
  AttendArgs a = a0;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.Hkv = Hkv;
  a.kv.hkv_m = hkv_m;
  a.cap = cap;
  a.chunk = chunk;
  __shared__ __attribute__((aligned(16))) float s_w[R][kMaxChunks];  // (rows read 16 bytes at a time)
  __shared__ float s_lc[R * (kMaxChunks + 1)];
  const int bg = blockIdx.y;
  const int b = div_by(bg, a.Hkv, a.kv.hkv_m);  // (a.kv.Hkv == a.Hkv)
  const int g = bg - b * a.Hkv;
  const int c = blockIdx.x;
  const int len = min(a.kv_len[b], a.cap);  // (kv_len <= capacity is a precondition; clamped all the same)
  const int nch_b = (max(len, 0) + a.chunk - 1) >> __builtin_ctz(a.chunk);  // (chunk is a power of two)
  const size_t bh0 = (size_t)b * a.Hq + (size_t)(g * R);
  if (nch_b == 0) {  // no cached position: attention over the empty set is the zero vector
    if (c == 0)
      for (int i = threadIdx.x; i < R * kHeadDim; i += kDenseWaves * 64) a.out[bh0 * kHeadDim + i] = 0.f;
    return;
  }
  if (c >= nch_b) return;
  unsigned long long* genp = a.ws_gen + bg;
  const unsigned long long gen = __hip_atomic_load(genp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int p0 = c * a.chunk;
  const int p1 = min(p0 + a.chunk, len);
  attend_rows<R, kPaged>(a, b, g, c, p0, p1 - p0);
  // (the tag of chunk t: pad words 2 and 3 of head 0's partial of chunk t)
  auto tag_at = [&](int t) {
    return reinterpret_cast<unsigned long long*>(a.ws_part + (bh0 * a.nch + (size_t)t) * kPartFloats + 2);
  };
  wait_memory();  // this thread's part of the partial has reached the point of coherence
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_store(tag_at(c), chunk_tag(gen, c), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_memory();
  }
  __syncthreads();
  bool ok = true;
  for (int t = threadIdx.x; t < nch_b; t += kDenseWaves * 64)
    ok = ok && __hip_atomic_load(tag_at(t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == chunk_tag(gen, t);
  if (!__syncthreads_and(ok)) return;
  combine_group<R, kDenseWaves * 64>(a.ws_part + bh0 * a.nch * kPartFloats, a.nch, nch_b, a.out + bh0 * kHeadDim,
                                     s_w, s_lc, genp, gen);
}

// --------------------------------------------------------------------------
// Launchers
// --------------------------------------------------------------------------

// Launch `kernel` as the i-th launch of a call; when this thread has profiling
// events for slot i, the dispatch records them around the kernel.
template <typename Kernel, typename... Args>
static void launch_k(int i, Kernel kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  const ProfileEvents& pe = profile_events();
  if (2 * i + 1 < pe.n)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, pe.ev[2 * i], pe.ev[2 * i + 1], 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

hipError_t launch_encode_keys(int B, const KvLayout& kv, const uint16_t* k, const int32_t* start,
                              const int32_t* end, uint8_t* codes, hipStream_t s, int max_rows) {
  const int bg = B * kv.Hkv;
  const int rows = max_rows > 0 && max_rows < kv.cap ? max_rows : kv.cap;
  int nblk = (rows + 63) / 64;
  const int cap_blocks = 2048 / bg > 0 ? 2048 / bg : 1;
  if (nblk > cap_blocks) nblk = cap_blocks;
  if (kv.table)
    launch_k(0, encode_keys_kernel<true>, dim3(nblk, bg), dim3(256), 0, s, k, start, end, codes, kv.Hkv, kv.hkv_m,
             kv.cap, kv);
  else
    launch_k(0, encode_keys_kernel<false>, dim3(nblk, bg), dim3(256), 0, s, k, start, end, codes, kv.Hkv, kv.hkv_m,
             kv.cap, kv);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_dense_r(const Plan& p, const KvLayout& kv, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const int32_t* kv_len, float scale, float* out, char* ws,
                                 hipStream_t s) {
  float* ws_part = reinterpret_cast<float*>(ws + p.off_part);
  auto* ws_gen = reinterpret_cast<unsigned long long*>(ws + p.off_count);
  AttendArgs aa{q, k, v, kv_len, ws_part, ws_gen, out, scale * 1.4426950408889634f, p.Hq, p.Hkv, p.cap, p.chunk,
                p.nch, kv};
  if (kv.table)
    launch_k(0, dense_attend_kernel<R, true>, dim3(p.nch, p.B * p.Hkv), dim3(kDenseWaves * 64), 0, s, aa.q, aa.k, aa.v,
             aa.kv_len, aa.Hkv, aa.kv.hkv_m, aa.cap, aa.chunk, aa);
  else
    launch_k(0, dense_attend_kernel<R, false>, dim3(p.nch, p.B * p.Hkv), dim3(kDenseWaves * 64), 0, s, aa.q, aa.k, aa.v,
             aa.kv_len, aa.Hkv, aa.kv.hkv_m, aa.cap, aa.chunk, aa);
  return hipGetLastError();
}

hipError_t launch_dense(const Plan& p, const KvLayout& kv, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int32_t* kv_len, float scale, float* out, char* ws,
                        hipStream_t s) {
  switch (p.R) {
    case 1: return launch_dense_r<1>(p, kv, q, k, v, kv_len, scale, out, ws, s);
    case 2: return launch_dense_r<2>(p, kv, q, k, v, kv_len, scale, out, ws, s);
    case 4: return launch_dense_r<4>(p, kv, q, k, v, kv_len, scale, out, ws, s);
    case 8: return launch_dense_r<8>(p, kv, q, k, v, kv_len, scale, out, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace adamas
