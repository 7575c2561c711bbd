// kernels.hip -- gfx950 kernels of the Adamas decode step.
//
// Method (sources by page title and section):
//   "Adamas: Hadamard Sparse Attention for Efficient Long-Context Inference",
//   v1/v2 abstracts: transform q and k with a Hadamard matrix, bucketize to 2-bit
//   codes, estimate similarity by Manhattan distance between codes, keep the
//   top-k positions under a token budget, gather the original K/V rows there and
//   run exact softmax attention over them.
//   "ADAMAS：稀疏注意力优化技术解析与应用实践" blog: section 2.2 (thresholds),
//   section 2.3 (integer Manhattan distance, popcount), section 3.1 (key codes kept
//   in a cache updated per appended key).
//
// Kernels (one decode step = scan -> select -> attend):
//   encode_keys_kernel  transform + bucketize + pack every key in [start, end)
//   scan_kernel         per (b, kv head, chunk): encode the group's queries,
//                       stream the packed key codes once, compute the distance of
//                       every key to each of the group's R query codes, keep the
//                       distances and a per-chunk histogram of them
//   select_kernel       per (b, q head): total histogram -> threshold distance T
//                       and the tie quota at T, then per-chunk output offsets and
//                       tie allowances (lower position wins ties)
//   attend_kernel       per (b, kv head, chunk): ordered compaction of the chunk's
//                       selected positions (sel_idx), gather of their K/V rows,
//                       exact softmax partials (m, l, o) per q head; the last
//                       block of each (b, kv head) merges the partials into out
//   The dense baseline reuses attend_kernel with every position selected,
//   followed by combine_kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "plan.h"

namespace adamas {

// --------------------------------------------------------------------------
// Key encode
// --------------------------------------------------------------------------

// grid (nblk, B*Hkv), 256 threads = 64 vectors per pass (a quad per vector).
__global__ __launch_bounds__(256) void encode_keys_kernel(const uint16_t* __restrict__ k,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ end,
                                                          uint8_t* __restrict__ codes, int Hkv, int cap) {
  const int bg = blockIdx.y;
  const int b = bg / Hkv;
  const int s = start ? start[b] : 0;
  const int e = end[b];
  const int quarter = threadIdx.x & 3;
  const int slot = threadIdx.x >> 2;  // 0..63
  const size_t base = (size_t)bg * (size_t)cap;
  // The loop bound depends only on blockIdx, so every quad runs every pass.
  for (int p0 = s + (int)blockIdx.x * 64; p0 < e; p0 += (int)gridDim.x * 64) {
    const int p = p0 + slot;
    const bool valid = p < e;
    const int pl = valid ? p : e - 1;  // clamped rows keep the loads in bounds
    const uint4* src = reinterpret_cast<const uint4*>(k + (base + (size_t)pl) * kHeadDim + quarter * 32);
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = src[i];
    float x[32];
    widen32(w, x);
    uint32_t lo, hi;
    encode_quad(x, quarter, lo, hi);
    if (valid) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + (base + (size_t)p) * kCodeBytes);
      dst[quarter] = lo;
      dst[4 + quarter] = hi;
    }
  }
}

// --------------------------------------------------------------------------
// Scan: Manhattan distance of packed 2-bit codes
// --------------------------------------------------------------------------
//
// Distance identity (derived here, not taken from the pages): with thermometer
// bits t1 = [c >= 1], t2 = [c >= 2], t3 = [c >= 3] of a code c = 2*hi + lo,
// |a - b| = [t1(a) != t1(b)] + [t2(a) != t2(b)] + [t3(a) != t3(b)], and
// t1 = lo | hi, t2 = hi, t3 = lo & hi.  On the planar layout one 32-bit word of
// each plane covers 32 coordinates, so a key costs 2 ops for its thermometer
// words plus, per query head, 3 XOR + 3 popcount per 32 coordinates.

struct ScanArgs {
  const uint16_t* q;
  const uint8_t* codes;
  const int32_t* kv_len;
  uint16_t* ws_dist;   // [B][Hkv][cap][R]
  uint16_t* ws_hist;   // [B][Hq][nch][kHistStride]
  uint16_t* dist_out;  // optional [B][Hq][cap]
  uint8_t* q_codes;    // optional [B][Hq][32]
  int Hq, Hkv, cap, chunk, nch;
};

template <int R>
__device__ __forceinline__ void store_dists(uint16_t* p, const uint32_t (&D)[R]) {
  if constexpr (R == 1) {
    p[0] = (uint16_t)D[0];
  } else if constexpr (R == 2) {
    *reinterpret_cast<uint32_t*>(p) = D[0] | (D[1] << 16);
  } else if constexpr (R == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(D[0] | (D[1] << 16), D[2] | (D[3] << 16));
  } else {
    *reinterpret_cast<uint4*>(p) =
        make_uint4(D[0] | (D[1] << 16), D[2] | (D[3] << 16), D[4] | (D[5] << 16), D[6] | (D[7] << 16));
  }
}

template <int R>
__device__ __forceinline__ void load_dists(const uint16_t* p, uint32_t (&D)[R]) {
  if constexpr (R == 1) {
    D[0] = p[0];
  } else if constexpr (R == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    D[0] = w & 0xFFFF;
    D[1] = w >> 16;
  } else if constexpr (R == 4) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    D[0] = w.x & 0xFFFF;
    D[1] = w.x >> 16;
    D[2] = w.y & 0xFFFF;
    D[3] = w.y >> 16;
  } else {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    D[0] = w.x & 0xFFFF;
    D[1] = w.x >> 16;
    D[2] = w.y & 0xFFFF;
    D[3] = w.y >> 16;
    D[4] = w.z & 0xFFFF;
    D[5] = w.z >> 16;
    D[6] = w.w & 0xFFFF;
    D[7] = w.w >> 16;
  }
}

// Encode the R query vectors of KV group (b, g) with wave 0 of the block and
// return their thermometer words through LDS (t1[4], t2[4], t3[4] per head).
template <int R>
__device__ __forceinline__ void encode_group_queries(const uint16_t* __restrict__ q, int b, int g, int Hq,
                                                     uint32_t (*s_qt)[12], uint8_t* q_codes) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int quarter = lane & 3;
    const int v = lane >> 2;
    const int vr = v < R ? v : R - 1;
    const int h = g * R + vr;
    const uint4* src =
        reinterpret_cast<const uint4*>(q + ((size_t)b * Hq + (size_t)h) * kHeadDim + quarter * 32);
    uint4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = src[i];
    float x[32];
    widen32(w, x);
    uint32_t lo, hi;
    encode_quad(x, quarter, lo, hi);
    if (v < R) {
      s_qt[v][quarter] = lo | hi;
      s_qt[v][4 + quarter] = hi;
      s_qt[v][8 + quarter] = lo & hi;
      if (q_codes) {
        uint32_t* d = reinterpret_cast<uint32_t*>(q_codes + ((size_t)b * Hq + (size_t)h) * kCodeBytes);
        d[quarter] = lo;
        d[4 + quarter] = hi;
      }
    }
  }
}

template <int R>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int c = blockIdx.x;
  const int len = a.kv_len[b];
  const int p0 = c * a.chunk;
  if (p0 >= len) return;
  const int p1 = min(p0 + a.chunk, len);
  const int tid = threadIdx.x;

  __shared__ uint32_t s_hist[R][kHistStride];
  __shared__ uint32_t s_qt[R][12];
  for (int i = tid; i < R * kHistStride; i += 256) (&s_hist[0][0])[i] = 0u;
  encode_group_queries<R>(a.q, b, g, a.Hq, s_qt, c == 0 ? a.q_codes : nullptr);
  __syncthreads();

  uint32_t qt[R][12];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 12; ++i) qt[r][i] = __builtin_amdgcn_readfirstlane(s_qt[r][i]);

  const uint4* cbase = reinterpret_cast<const uint4*>(a.codes + (size_t)bg * (size_t)a.cap * kCodeBytes);
  uint16_t* dws = a.ws_dist + (size_t)bg * (size_t)a.cap * R;
  constexpr int KB = 4;  // keys per thread per pass
  for (int base = p0; base < p1; base += KB * 256) {
    uint4 klo[KB], khi[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int p = base + i * 256 + tid;
      if (p < p1) {
        klo[i] = cbase[(size_t)p * 2];
        khi[i] = cbase[(size_t)p * 2 + 1];
      }
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int p = base + i * 256 + tid;
      if (p < p1) {
        const uint32_t lo[4] = {klo[i].x, klo[i].y, klo[i].z, klo[i].w};
        const uint32_t hi[4] = {khi[i].x, khi[i].y, khi[i].z, khi[i].w};
        uint32_t t1[4], t3[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          t1[w] = lo[w] | hi[w];
          t3[w] = lo[w] & hi[w];
        }
        uint32_t D[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t d = 0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            d += __builtin_popcount(t1[w] ^ qt[r][w]);
            d += __builtin_popcount(hi[w] ^ qt[r][4 + w]);
            d += __builtin_popcount(t3[w] ^ qt[r][8 + w]);
          }
          D[r] = d;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) atomicAdd(&s_hist[r][D[r]], 1u);
        store_dists<R>(dws + (size_t)p * R, D);
        if (a.dist_out) {
#pragma unroll
          for (int r = 0; r < R; ++r)
            a.dist_out[((size_t)b * a.Hq + (size_t)(g * R + r)) * (size_t)a.cap + p] = (uint16_t)D[r];
        }
      }
    }
  }
  __syncthreads();
  uint16_t* hout = a.ws_hist + ((size_t)(b * a.Hq + g * R) * a.nch + c) * kHistStride;
  for (int i = tid; i < R * kHistStride; i += 256) {
    const int r = i / kHistStride;
    const int d = i - r * kHistStride;
    hout[(size_t)r * a.nch * kHistStride + d] = (uint16_t)s_hist[r][d];
  }
}

// --------------------------------------------------------------------------
// Select: threshold distance and per-chunk offsets
// --------------------------------------------------------------------------

struct SelectArgs {
  const int32_t* kv_len;
  const uint16_t* ws_hist;  // [B][Hq][nch][kHistStride]
  int2* ws_cinfo;           // [B][Hq][nch]: {output offset, ties to take}
  int2* ws_hinfo;           // [B][Hq]: {T, k_eff}
  uint32_t* counters;       // [B][Hkv]
  int32_t* sel_idx;         // optional
  int Hq, Hkv, R, budget, chunk, nch;
};

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// grid (B*Hq), 256 threads, dynamic LDS = nch * kHistStride * 2 bytes.
__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int len = a.kv_len[b];
  const int k_eff = min(a.budget, len);
  const int nch_b = (len + a.chunk - 1) / a.chunk;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();

  extern __shared__ uint4 s_dyn[];
  uint16_t* s_h = reinterpret_cast<uint16_t*>(s_dyn);  // [nch_b][kHistStride]
  __shared__ uint32_t s_tot[kHistStride];
  __shared__ uint32_t s_lt[kMaxChunks], s_eq[kMaxChunks];
  __shared__ int s_T;
  __shared__ uint32_t s_quota;

  const uint4* src = reinterpret_cast<const uint4*>(a.ws_hist + (size_t)bh * a.nch * kHistStride);
  const int n16 = nch_b * (kHistStride * 2 / 16);
  for (int i = tid; i < n16; i += 256) s_dyn[i] = src[i];
  __syncthreads();

  for (int d = tid; d < kBins; d += 256) {
    uint32_t s = 0;
    for (int c = 0; c < nch_b; ++c) s += s_h[c * kHistStride + d];
    s_tot[d] = s;
  }
  __syncthreads();

  if (wave == 0) {
    // lane covers bins [7*lane, 7*lane + 7) of 0..384
    uint32_t loc = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int d = 7 * lane + j;
      if (d < kBins) loc += s_tot[d];
    }
    uint32_t inc = loc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(inc, off, 64);
      if (lane >= off) inc += t;
    }
    const uint64_t ball = __ballot(inc >= (uint32_t)k_eff);
    const int first = __builtin_ffsll((long long)ball) - 1;  // exists: the total is len >= k_eff
    if (lane == first) {
      uint32_t cum = inc - loc;
      int T = 7 * lane;
      for (int j = 0; j < 7; ++j) {
        const int d = 7 * lane + j;
        const uint32_t nc = cum + s_tot[d];
        if (nc >= (uint32_t)k_eff) {
          T = d;
          break;
        }
        cum = nc;
      }
      s_T = T;
      s_quota = (uint32_t)k_eff - cum;
    }
  }
  __syncthreads();
  const int T = s_T;
  const uint32_t quota = s_quota;

  for (int c = wave; c < nch_b; c += 4) {
    uint32_t s = 0;
    for (int d = lane; d < T; d += 64) s += s_h[c * kHistStride + d];
    s = wave_sum_u32(s);
    if (lane == 0) {
      s_lt[c] = s;
      s_eq[c] = s_h[c * kHistStride + T];
    }
  }
  __syncthreads();

  if (wave == 0) {
    // two chunks per lane: c0 = 2*lane, c1 = 2*lane + 1 (nch_b <= 128)
    const int c0 = 2 * lane, c1 = 2 * lane + 1;
    const uint32_t eq0 = c0 < nch_b ? s_eq[c0] : 0u, eq1 = c1 < nch_b ? s_eq[c1] : 0u;
    const uint32_t lt0 = c0 < nch_b ? s_lt[c0] : 0u, lt1 = c1 < nch_b ? s_lt[c1] : 0u;
    uint32_t inc = eq0 + eq1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(inc, off, 64);
      if (lane >= off) inc += t;
    }
    const uint32_t E0 = inc - (eq0 + eq1);
    const uint32_t E1 = E0 + eq0;
    const uint32_t take0 = quota > E0 ? min(quota - E0, eq0) : 0u;
    const uint32_t take1 = quota > E1 ? min(quota - E1, eq1) : 0u;
    const uint32_t sel0 = lt0 + take0, sel1 = lt1 + take1;
    uint32_t sinc = sel0 + sel1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(sinc, off, 64);
      if (lane >= off) sinc += t;
    }
    const uint32_t S0 = sinc - (sel0 + sel1);
    int2* ci = a.ws_cinfo + (size_t)bh * a.nch;
    if (c0 < nch_b) ci[c0] = make_int2((int)S0, (int)take0);
    if (c1 < nch_b) ci[c1] = make_int2((int)(S0 + sel0), (int)take1);
  }
  if (tid == 0) {
    a.ws_hinfo[bh] = make_int2(T, k_eff);
    if (h % a.R == 0) a.counters[b * a.Hkv + h / a.R] = 0u;
  }
  if (a.sel_idx) {
    for (int i = k_eff + tid; i < a.budget; i += 256) a.sel_idx[(size_t)bh * a.budget + i] = -1;
  }
}

// --------------------------------------------------------------------------
// Attend: compaction, gather and exact softmax partials
// --------------------------------------------------------------------------

struct AttendArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  const uint16_t* ws_dist;
  const int2* ws_cinfo;
  const int2* ws_hinfo;
  float* ws_part;       // [B][Hq][nch][kPartFloats]
  uint32_t* counters;   // [B][Hkv] (sparse path only)
  int32_t* sel_idx;     // optional
  float* out;
  float qscale;         // softmax scale * log2(e)
  int Hq, Hkv, cap, budget, chunk, nch;
};

// Merge the per-chunk partials of one (b, q head) into out.
__device__ __forceinline__ void combine_partials(const float* __restrict__ part, int nch_b, int d,
                                                 float* __restrict__ out_row) {
  float M = -INFINITY;
  for (int c = 0; c < nch_b; ++c) M = fmaxf(M, part[(size_t)c * kPartFloats]);
  float L = 0.f, O = 0.f;
  for (int c = 0; c < nch_b; ++c) {
    const float* pc = part + (size_t)c * kPartFloats;
    const float mc = pc[0];
    if (mc != -INFINITY) {
      const float w = exp2f(mc - M);
      L = __builtin_fmaf(pc[1], w, L);
      O = __builtin_fmaf(pc[4 + d], w, O);
    }
  }
  out_row[d] = O / L;
}

template <int R, bool DENSE>
__global__ __launch_bounds__(256) void attend_kernel(AttendArgs a) {
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int c = blockIdx.x;
  const int len = a.kv_len[b];
  const int nch_b = (len + a.chunk - 1) / a.chunk;
  if (c >= nch_b) return;
  const int p0 = c * a.chunk;
  const int p1 = min(p0 + a.chunk, len);
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();

  __shared__ float s_q[R][kHeadDim];
  __shared__ int s_pos[DENSE ? 1 : kMaxChunk];
  __shared__ uint8_t s_mask[DENSE ? 1 : kMaxChunk];
  __shared__ int s_cnt[4][2 * R + 1];
  __shared__ float s_m[4][R], s_l[4][R];
  __shared__ float s_o[4][R][kHeadDim];
  __shared__ int s_last;

  for (int i = tid; i < R * kHeadDim; i += 256) {
    const int r = i / kHeadDim, d = i - r * kHeadDim;
    const uint16_t bits = a.q[((size_t)b * a.Hq + (size_t)(g * R + r)) * kHeadDim + d];
    s_q[r][d] = __uint_as_float((uint32_t)bits << 16) * a.qscale;
  }

  int nrows;
  if constexpr (DENSE) {
    nrows = p1 - p0;
  } else {
    int T[R], take[R], S[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const size_t bh = (size_t)b * a.Hq + (size_t)(g * R + r);
      T[r] = a.ws_hinfo[bh].x;
      const int2 ci = a.ws_cinfo[bh * a.nch + c];
      S[r] = ci.x;
      take[r] = ci.y;
    }
    int carry_eq[R], carry_sel[R];
#pragma unroll
    for (int r = 0; r < R; ++r) carry_eq[r] = carry_sel[r] = 0;
    int carry_u = 0;
    const uint16_t* dws = a.ws_dist + (size_t)bg * (size_t)a.cap * R;
    for (int base = p0; base < p1; base += 256) {
      const int p = base + tid;
      const bool valid = p < p1;
      uint32_t D[R];
      if (valid) {
        load_dists<R>(dws + (size_t)p * R, D);
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) D[r] = 0xFFFFu;
      }
      // ranks among the ties at T, in position order
      uint64_t beq[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        beq[r] = __ballot(valid && D[r] == (uint32_t)T[r]);
        if (lane == 0) s_cnt[wave][r] = __builtin_popcountll(beq[r]);
      }
      __syncthreads();
      bool sel[R];
      uint32_t mask = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int before = carry_eq[r] + (int)lanes_below(beq[r]);
        int tot = 0;
        for (int w = 0; w < 4; ++w) {
          if (w < wave) before += s_cnt[w][r];
          tot += s_cnt[w][r];
        }
        carry_eq[r] += tot;
        const bool is_eq = valid && D[r] == (uint32_t)T[r];
        sel[r] = (valid && D[r] < (uint32_t)T[r]) || (is_eq && before < take[r]);
        mask |= (sel[r] ? 1u : 0u) << r;
      }
      __syncthreads();
      uint64_t bsel[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        bsel[r] = __ballot(sel[r]);
        if (lane == 0) s_cnt[wave][R + r] = __builtin_popcountll(bsel[r]);
      }
      const uint64_t bu = __ballot(mask != 0);
      if (lane == 0) s_cnt[wave][2 * R] = __builtin_popcountll(bu);
      __syncthreads();
#pragma unroll
      for (int r = 0; r < R; ++r) {
        int before = carry_sel[r] + (int)lanes_below(bsel[r]);
        int tot = 0;
        for (int w = 0; w < 4; ++w) {
          if (w < wave) before += s_cnt[w][R + r];
          tot += s_cnt[w][R + r];
        }
        if (sel[r] && a.sel_idx)
          a.sel_idx[((size_t)b * a.Hq + (size_t)(g * R + r)) * a.budget + S[r] + before] = p;
        carry_sel[r] += tot;
      }
      {
        int before = carry_u + (int)lanes_below(bu);
        int tot = 0;
        for (int w = 0; w < 4; ++w) {
          if (w < wave) before += s_cnt[w][2 * R];
          tot += s_cnt[w][2 * R];
        }
        if (mask) {
          s_pos[before] = p;
          s_mask[before] = (uint8_t)mask;
        }
        carry_u += tot;
      }
      __syncthreads();
    }
    nrows = carry_u;
  }
  __syncthreads();

  // Online softmax over the gathered rows: wave w takes rows w, w+4, ...; lane
  // holds dims 2*lane, 2*lane+1.
  float q0[R], q1[R], m[R], l[R], o0[R], o1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    q0[r] = s_q[r][2 * lane];
    q1[r] = s_q[r][2 * lane + 1];
    m[r] = -INFINITY;
    l[r] = 0.f;
    o0[r] = 0.f;
    o1[r] = 0.f;
  }
  const uint32_t* Kb = reinterpret_cast<const uint32_t*>(a.k + (size_t)bg * (size_t)a.cap * kHeadDim);
  const uint32_t* Vb = reinterpret_cast<const uint32_t*>(a.v + (size_t)bg * (size_t)a.cap * kHeadDim);
  constexpr int U = 4;  // rows in flight per wave
  for (int i0 = wave; i0 < nrows; i0 += 4 * U) {
    uint32_t kw[U], vw[U], mk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 4 * u;
      if (i < nrows) {
        int p;
        if constexpr (DENSE) {
          p = p0 + i;
          mk[u] = (1u << R) - 1u;
        } else {
          p = s_pos[i];
          mk[u] = s_mask[i];
        }
        kw[u] = Kb[(size_t)p * 64 + lane];
        vw[u] = Vb[(size_t)p * 64 + lane];
      } else {
        mk[u] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (mk[u] == 0u) continue;
      const float k0 = bf16_lo(kw[u]), k1 = bf16_hi(kw[u]);
      const float v0 = bf16_lo(vw[u]), v1 = bf16_hi(vw[u]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (mk[u] & (1u << r)) {
          const float s = wave_sum(__builtin_fmaf(q0[r], k0, q1[r] * k1));
          const float mn = fmaxf(m[r], s);
          const float corr = exp2f(m[r] - mn);
          const float pr = exp2f(s - mn);
          l[r] = __builtin_fmaf(l[r], corr, pr);
          o0[r] = __builtin_fmaf(o0[r], corr, pr * v0);
          o1[r] = __builtin_fmaf(o1[r], corr, pr * v1);
          m[r] = mn;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (lane == 0) {
      s_m[wave][r] = m[r];
      s_l[wave][r] = l[r];
    }
    s_o[wave][r][2 * lane] = o0[r];
    s_o[wave][r][2 * lane + 1] = o1[r];
  }
  __syncthreads();
  for (int i = tid; i < R * kHeadDim; i += 256) {
    const int r = i / kHeadDim, d = i - r * kHeadDim;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][r]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (s_m[w][r] != -INFINITY) {
          const float f = exp2f(s_m[w][r] - M);
          L = __builtin_fmaf(s_l[w][r], f, L);
          O = __builtin_fmaf(s_o[w][r][d], f, O);
        }
      }
    }
    float* pc = a.ws_part + (((size_t)b * a.Hq + (size_t)(g * R + r)) * a.nch + c) * kPartFloats;
    if (d == 0) {
      pc[0] = M;
      pc[1] = L;
    }
    pc[4 + d] = O;
  }

  if constexpr (!DENSE) {
    // The last block of this (b, kv head) to finish merges every chunk's partials.
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&a.counters[bg], 1u) == (uint32_t)(nch_b - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int i = tid; i < R * kHeadDim; i += 256) {
      const int r = i / kHeadDim, d = i - r * kHeadDim;
      const size_t bh = (size_t)b * a.Hq + (size_t)(g * R + r);
      combine_partials(a.ws_part + bh * a.nch * kPartFloats, nch_b, d, a.out + bh * kHeadDim);
    }
  }
}

// Dense path: one block per (b, q head), 128 threads.
__global__ __launch_bounds__(128) void combine_kernel(const float* __restrict__ part, const int32_t* kv_len,
                                                      float* __restrict__ out, int Hq, int chunk, int nch) {
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int nch_b = (kv_len[b] + chunk - 1) / chunk;
  combine_partials(part + (size_t)bh * nch * kPartFloats, nch_b, threadIdx.x, out + (size_t)bh * kHeadDim);
}

// --------------------------------------------------------------------------
// Launchers
// --------------------------------------------------------------------------

hipError_t launch_encode_keys(int B, int Hkv, int cap, const uint16_t* k, const int32_t* start,
                              const int32_t* end, uint8_t* codes, hipStream_t s) {
  const int bg = B * Hkv;
  int nblk = (cap + 63) / 64;
  const int cap_blocks = 2048 / bg > 0 ? 2048 / bg : 1;
  if (nblk > cap_blocks) nblk = cap_blocks;
  hipLaunchKernelGGL(encode_keys_kernel, dim3(nblk, bg), dim3(256), 0, s, k, start, end, codes, Hkv, cap);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_decode_r(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const uint8_t* codes, const int32_t* kv_len, float scale, float* out,
                                  int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, char* ws, hipStream_t s) {
  uint16_t* ws_dist = reinterpret_cast<uint16_t*>(ws + p.off_dist);
  uint16_t* ws_hist = reinterpret_cast<uint16_t*>(ws + p.off_hist);
  int2* ws_cinfo = reinterpret_cast<int2*>(ws + p.off_cinfo);
  int2* ws_hinfo = reinterpret_cast<int2*>(ws + p.off_hinfo);
  float* ws_part = reinterpret_cast<float*>(ws + p.off_part);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + p.off_count);
  const dim3 grid_chunks(p.nch, p.B * p.Hkv);

  ScanArgs sa{q, codes, kv_len, ws_dist, ws_hist, dist, q_codes, p.Hq, p.Hkv, p.cap, p.chunk, p.nch};
  hipLaunchKernelGGL(scan_kernel<R>, grid_chunks, dim3(256), 0, s, sa);

  SelectArgs la{kv_len, ws_hist, ws_cinfo, ws_hinfo, counters, sel_idx, p.Hq, p.Hkv, R, p.budget, p.chunk, p.nch};
  const size_t lds = (size_t)p.nch * kHistStride * sizeof(uint16_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(select_kernel, dim3(p.B * p.Hq), dim3(256), lds, s, la);

  AttendArgs aa{q,        k,       v,   kv_len,    ws_dist, ws_cinfo, ws_hinfo, ws_part, counters,
                sel_idx,  out,     scale * 1.4426950408889634f, p.Hq, p.Hkv, p.cap, p.budget, p.chunk, p.nch};
  hipLaunchKernelGGL((attend_kernel<R, false>), grid_chunks, dim3(256), 0, s, aa);
  return hipGetLastError();
}

hipError_t launch_decode(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint8_t* codes, const int32_t* kv_len, float scale, float* out,
                         int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, char* ws, hipStream_t s) {
  switch (p.R) {
    case 1: return launch_decode_r<1>(p, q, k, v, codes, kv_len, scale, out, sel_idx, dist, q_codes, ws, s);
    case 2: return launch_decode_r<2>(p, q, k, v, codes, kv_len, scale, out, sel_idx, dist, q_codes, ws, s);
    case 4: return launch_decode_r<4>(p, q, k, v, codes, kv_len, scale, out, sel_idx, dist, q_codes, ws, s);
    case 8: return launch_decode_r<8>(p, q, k, v, codes, kv_len, scale, out, sel_idx, dist, q_codes, ws, s);
    default: return hipErrorInvalidValue;
  }
}

template <int R>
static hipError_t launch_dense_r(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* kv_len, float scale, float* out, char* ws, hipStream_t s) {
  float* ws_part = reinterpret_cast<float*>(ws + p.off_part);
  AttendArgs aa{q,       k,       v,       kv_len, nullptr, nullptr, nullptr, ws_part, nullptr,
                nullptr, out,     scale * 1.4426950408889634f, p.Hq, p.Hkv, p.cap, 0, p.chunk, p.nch};
  hipLaunchKernelGGL((attend_kernel<R, true>), dim3(p.nch, p.B * p.Hkv), dim3(256), 0, s, aa);
  hipLaunchKernelGGL(combine_kernel, dim3(p.B * p.Hq), dim3(128), 0, s, ws_part, kv_len, out, p.Hq, p.chunk,
                     p.nch);
  return hipGetLastError();
}

hipError_t launch_dense(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* kv_len, float scale, float* out, char* ws, hipStream_t s) {
  switch (p.R) {
    case 1: return launch_dense_r<1>(p, q, k, v, kv_len, scale, out, ws, s);
    case 2: return launch_dense_r<2>(p, q, k, v, kv_len, scale, out, ws, s);
    case 4: return launch_dense_r<4>(p, q, k, v, kv_len, scale, out, ws, s);
    case 8: return launch_dense_r<8>(p, q, k, v, kv_len, scale, out, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace adamas
