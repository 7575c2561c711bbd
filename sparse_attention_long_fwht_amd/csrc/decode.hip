// decode.hip -- the Adamas decode step on gfx950: two kernels.
//
// Method (sources by page title and section):
//   "Adamas: Hadamard Sparse Attention for Efficient Long-Context Inference",
//   v1/v2 abstracts: Hadamard-transform q, bucketize to 2-bit codes, score every
//   cached key by the Manhattan distance between codes, keep the top-k positions
//   under a token budget, gather the original K/V rows there and run exact
//   softmax attention over them.
//   "ADAMAS：稀疏注意力优化技术解析与应用实践" blog, section 2.2 (thresholds -t, 0,
//   +t, t = max|y|/2, strict "<"), section 2.3 (integer Manhattan distance).
//
// scan_kernel          grid (chunks, B*Hkv): the group's R query vectors are
//                      encoded (one wave per vector), then each key code of the
//                      chunk is read once and its distance to all R query codes
//                      computed; distances go to a per-head array and a per-chunk
//                      histogram of them (0..384) to the workspace.
// select_attend_kernel grid (B*Hq, splits): per query head, the chunk histograms
//                      give the threshold distance T (the k-th smallest) and how
//                      many ties at T to keep; one ordered pass over the head's
//                      distances compacts the selected positions (every distance
//                      below T, then ties by ascending position) into LDS; the
//                      block gathers those K/V rows and runs exact softmax
//                      attention (MFMA for q.K, VALU for P.V).  With several
//                      splits each block takes a slice of the selection and the
//                      last one merges the slices' (m, l, o) partials.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "plan.h"

namespace adamas {

// --------------------------------------------------------------------------
// Query encode, one 128-vector per wave
// --------------------------------------------------------------------------
//
// Lane l holds coordinates l and l + 64.  Butterflies of half-width 1..32 pair
// lane l with lane l ^ h (each output = one fp32 add or subtract of the same two
// operands as the stage-by-stage transform: fma with a +-1 multiplier rounds
// once); half-width 64 pairs the two registers of a lane.  Stage order
// 1, 2, 4, ..., 64 as everywhere else.  The codes come out as wave ballots: bit l
// of a ballot over coordinate l is exactly the planar packed layout.

template <int H>
__device__ __forceinline__ float xor_partner(float v) {
  if constexpr (H == 1) return quad_swap<kQuadXor1>(v);
  else if constexpr (H == 2) return quad_swap<kQuadXor2>(v);
  else if constexpr (H < 32) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (H << 10)));
  else return __shfl_xor(v, 32, 64);
}

template <int H>
__device__ __forceinline__ void wave_butterfly(float& x0, float& x1, int lane) {
  const float sgn = (lane & H) ? -1.0f : 1.0f;
  const float p0 = xor_partner<H>(x0);
  const float p1 = xor_partner<H>(x1);
  x0 = __builtin_fmaf(x0, sgn, p0);
  x1 = __builtin_fmaf(x1, sgn, p1);
}

// qbits: the bf16 values of coordinates l and l + 64 in the low/high 16 bits.
// Returns the code as dwords: lo[0..3] = low-bit plane, hi[0..3] = high-bit plane
// (wave-uniform values).
__device__ __forceinline__ void encode_wave(uint32_t qlo_bits, uint32_t qhi_bits, uint32_t (&lo)[4],
                                            uint32_t (&hi)[4]) {
  const int lane = lane_id();
  float x0 = __uint_as_float(qlo_bits << 16);
  float x1 = __uint_as_float(qhi_bits << 16);
  wave_butterfly<1>(x0, x1, lane);
  wave_butterfly<2>(x0, x1, lane);
  wave_butterfly<4>(x0, x1, lane);
  wave_butterfly<8>(x0, x1, lane);
  wave_butterfly<16>(x0, x1, lane);
  wave_butterfly<32>(x0, x1, lane);
  {
    const float a = x0, b = x1;
    x0 = a + b;
    x1 = a - b;
  }
  const float m = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float t = 0.5f * m;
  // code = [y >= -t] + [y >= 0] + [y >= t]: low bit = XOR of the three, high = [y >= 0]
  const bool l0 = !((x0 < -t) ^ (x0 < 0.0f) ^ (x0 < t));
  const bool l1 = !((x1 < -t) ^ (x1 < 0.0f) ^ (x1 < t));
  const uint64_t blo0 = __ballot(l0), blo1 = __ballot(l1);
  const uint64_t bhi0 = __ballot(!(x0 < 0.0f)), bhi1 = __ballot(!(x1 < 0.0f));
  lo[0] = (uint32_t)blo0;
  lo[1] = (uint32_t)(blo0 >> 32);
  lo[2] = (uint32_t)blo1;
  lo[3] = (uint32_t)(blo1 >> 32);
  hi[0] = (uint32_t)bhi0;
  hi[1] = (uint32_t)(bhi0 >> 32);
  hi[2] = (uint32_t)bhi1;
  hi[3] = (uint32_t)(bhi1 >> 32);
}

// --------------------------------------------------------------------------
// Scan
// --------------------------------------------------------------------------

constexpr int kScanThreads = 512;  // one key per thread per pass

struct ScanArgs {
  const uint16_t* q;
  const uint16_t* k;   // read only when `append`
  uint8_t* codes;      // written only when `append` (the appended key's code)
  const int32_t* kv_len;
  uint16_t* dist;      // [B][Hq][dstride] (workspace)
  uint16_t* dist_out;  // optional [B][Hq][cap]
  uint16_t* hist;      // [B][Hq][nch][kHistStride]
  uint8_t* q_codes;    // optional [B][Hq][32]
  uint32_t* counters;  // [B][Hq], cleared here for select_attend_kernel
  int Hq, Hkv, cap, dstride, chunk, nch, append;
};

template <int R>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(ScanArgs a) {
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int c = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int p0 = c * a.chunk;

  // first pass of key codes, addresses clamped to the capacity so that they
  // do not wait for kv_len
  const uint4* cbase = reinterpret_cast<const uint4*>(a.codes + (size_t)bg * (size_t)a.cap * kCodeBytes);
  int p = min(p0 + tid, a.cap - 1);
  uint4 klo = cbase[(size_t)p * 2];
  uint4 khi = cbase[(size_t)p * 2 + 1];
  const int len = a.kv_len[b];

  __shared__ uint32_t s_hist[R][kHistStride];
  __shared__ uint32_t s_code[R + 1][8];  // query codes, then the appended key's
  for (int i = tid; i < R * kHistStride; i += kScanThreads) (&s_hist[0][0])[i] = 0u;
  // Vectors to encode: the group's R queries, plus -- in the block holding
  // position len-1 when appending -- that key.  Wave w takes vectors w, w+8.
  const bool app_here = a.append && (len - 1) >= p0 && (len - 1) < p0 + a.chunk;
  const int nvec = R + (app_here ? 1 : 0);
#pragma unroll 1
  for (int vi = wave; vi < nvec; vi += kScanThreads / 64) {
    const uint16_t* row = vi < R ? a.q + ((size_t)b * a.Hq + (size_t)(g * R + vi)) * kHeadDim
                                 : a.k + ((size_t)bg * a.cap + (size_t)(len - 1)) * kHeadDim;
    uint32_t lo[4], hi[4];
    encode_wave(row[lane], row[lane + 64], lo, hi);
    if (lane < 8) {
      const uint32_t w = lane < 4 ? lo[lane & 3] : hi[lane & 3];
      s_code[vi][lane] = w;
      if (vi < R) {
        if (c == 0 && a.q_codes)
          reinterpret_cast<uint32_t*>(a.q_codes + ((size_t)b * a.Hq + (size_t)(g * R + vi)) * kCodeBytes)[lane] = w;
      } else {
        reinterpret_cast<uint32_t*>(a.codes + ((size_t)bg * a.cap + (size_t)(len - 1)) * kCodeBytes)[lane] = w;
      }
    }
  }
  if (c == 0 && tid < R) a.counters[(size_t)b * a.Hq + g * R + tid] = 0u;
  __syncthreads();
  if (p0 >= len) return;
  const int p1 = min(p0 + a.chunk, len);

  // thermometer words of the query codes: t1 = lo|hi, t2 = hi, t3 = lo&hi
  uint32_t qt[R][12];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = __builtin_amdgcn_readfirstlane(s_code[r][w]);
      const uint32_t hi = __builtin_amdgcn_readfirstlane(s_code[r][4 + w]);
      qt[r][w] = lo | hi;
      qt[r][4 + w] = hi;
      qt[r][8 + w] = lo & hi;
    }

  uint16_t* drow = a.dist + ((size_t)b * a.Hq + (size_t)g * R) * (size_t)a.dstride;
#pragma unroll 1
  for (int base = p0; base < p1; base += kScanThreads) {
    if (base != p0) {
      p = min(base + tid, p1 - 1);
      klo = cbase[(size_t)p * 2];
      khi = cbase[(size_t)p * 2 + 1];
    }
    p = base + tid;
    if (p < p1) {
      if (app_here && p == len - 1) {  // the code this block just produced
        klo = make_uint4(s_code[R][0], s_code[R][1], s_code[R][2], s_code[R][3]);
        khi = make_uint4(s_code[R][4], s_code[R][5], s_code[R][6], s_code[R][7]);
      }
      // |a - b| summed over coordinates = popcount of the three thermometer
      // XORs (t1 = lo|hi, t2 = hi, t3 = lo&hi) over the 128 coordinates
      const uint32_t lo[4] = {klo.x, klo.y, klo.z, klo.w};
      const uint32_t hi[4] = {khi.x, khi.y, khi.z, khi.w};
      uint32_t t1[4], t3[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        t1[w] = lo[w] | hi[w];
        t3[w] = lo[w] & hi[w];
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t d = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          d += __builtin_popcount(t1[w] ^ qt[r][w]);
          d += __builtin_popcount(hi[w] ^ qt[r][4 + w]);
          d += __builtin_popcount(t3[w] ^ qt[r][8 + w]);
        }
        atomicAdd(&s_hist[r][d], 1u);
        drow[(size_t)r * a.dstride + p] = (uint16_t)d;
        if (a.dist_out) a.dist_out[((size_t)b * a.Hq + (size_t)(g * R + r)) * (size_t)a.cap + p] = (uint16_t)d;
      }
    }
  }
  __syncthreads();
  // histogram rows as u16 pairs
  uint32_t* hout = reinterpret_cast<uint32_t*>(a.hist + ((size_t)(b * a.Hq + g * R) * a.nch + c) * kHistStride);
  constexpr int W = kHistStride / 2;
  for (int i = tid; i < R * W; i += kScanThreads) {
    const int r = i / W;
    const int j = i - r * W;
    hout[(size_t)r * a.nch * W + j] = s_hist[r][2 * j] | (s_hist[r][2 * j + 1] << 16);
  }
}

// --------------------------------------------------------------------------
// Select + gather + attention
// --------------------------------------------------------------------------

struct SelAttArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  const uint16_t* dist;  // [B][Hq][dstride]
  const uint16_t* hist;  // [B][Hq][nch][kHistStride]
  float* part;           // [B][Hq][splits][kPartFloats]
  uint32_t* counters;    // [B][Hq]
  int32_t* sel_idx;      // optional [B][Hq][budget]
  float* out;            // [B][Hq][128]
  float qscale;          // softmax scale * log2(e)
  int Hq, Hkv, R, cap, dstride, budget, chunk, nch, splits, rows_per_split;
};

constexpr int kSAThreads = 512;
constexpr int kSAWaves = kSAThreads / 64;
constexpr int kSAPPT = 64;                       // positions per thread per pass
constexpr int kSAPass = kSAThreads * kSAPPT;     // 32768 positions per pass
constexpr int kSATile = kSAWaves * 16;           // 128 rows per attention tile

// Exclusive prefix sum over the block; `total` = block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wsum, uint32_t& total) {
  const int lane = lane_id(), wave = wave_id();
  const uint32_t inc = wave_inclusive_scan_u32(v);
  if (lane == 63) s_wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSAWaves; ++w) {
    const uint32_t x = s_wsum[w];
    before += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Number of the two 16-bit distances in w that are >= the threshold whose
// bias (0x8000 - thr in both halves) is given: d + 0x8000 - thr has its top
// bit set exactly when d >= thr (all values < 0x8000, so nothing wraps).
__device__ __forceinline__ uint32_t count_ge2(uint32_t w, uint32_t bias) {
  const u16x2_t s = __builtin_bit_cast(u16x2_t, w) + __builtin_bit_cast(u16x2_t, bias);
  return __builtin_popcount(__builtin_bit_cast(uint32_t, s) & 0x80008000u);
}

// Distances of the 16-byte word `i` of the 64 positions a thread owns, with
// positions at or past `len` replaced by 0x7FFF (never selected).
__device__ __forceinline__ uint4 masked_dists(uint4 w, int pos, int len) {
  uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = pos + 2 * j;
    if (p >= len) x[j] = 0x7FFF7FFFu;
    else if (p + 1 >= len) x[j] = (x[j] & 0xFFFFu) | 0x7FFF0000u;
  }
  return make_uint4(x[0], x[1], x[2], x[3]);
}

__global__ __launch_bounds__(kSAThreads) void select_attend_kernel(SelAttArgs a) {
  const int bh = blockIdx.x;
  const int split = blockIdx.y;
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / a.R;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();

  extern __shared__ int s_list[];  // this split's selected positions, in order
  __shared__ uint32_t s_tot[2][kHistStride];
  __shared__ uint32_t s_wsum[kSAWaves];
  __shared__ int s_T;
  __shared__ uint32_t s_quota;
  __shared__ float s_S[kSATile];
  __shared__ float s_m, s_l, s_corr;
  __shared__ float s_red[kSAWaves][kHeadDim];
  __shared__ int s_last;

  // ---- 1. loads: the first pass of distances, the chunk histograms (two
  // threads per bin pair: even / odd chunks), kv_len and the query fragment.
  const uint4* drow = reinterpret_cast<const uint4*>(a.dist + (size_t)bh * a.dstride);
  const int dmax16 = a.dstride / 8 - 1;  // last 16-byte word of the row
  uint4 dw[kSAPPT / 8];
#pragma unroll
  for (int i = 0; i < kSAPPT / 8; ++i) dw[i] = drow[min(tid * (kSAPPT / 8) + i, dmax16)];
  const int len = a.kv_len[b];
  const uint32_t* hbase = reinterpret_cast<const uint32_t*>(a.hist + (size_t)bh * a.nch * kHistStride);
  constexpr int W = kHistStride / 2;  // bin pairs per row
  const int hj = tid % W;
  const int hs = tid / W;  // 0, 1 for tid < 2W; larger values are idle
  const int col = lane & 15;
  const int kg = lane >> 4;
  uint4 qf[4];
  {
    const uint16_t* qrow = a.q + (size_t)bh * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = col == 0 ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * kg) : make_uint4(0, 0, 0, 0);
  }
  if (hs < 2) {
    const int nch_b = (len + a.chunk - 1) / a.chunk;
    uint32_t acc_lo = 0, acc_hi = 0;
#pragma unroll 1
    for (int c0 = hs; c0 < a.nch; c0 += 32) {
      uint32_t w[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) w[u] = hbase[(size_t)min(c0 + 2 * u, a.nch - 1) * W + hj];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const bool ok = c0 + 2 * u < nch_b;
        acc_lo += ok ? (w[u] & 0xFFFFu) : 0u;
        acc_hi += ok ? (w[u] >> 16) : 0u;
      }
    }
    s_tot[hs][2 * hj] = acc_lo;
    s_tot[hs][2 * hj + 1] = acc_hi;
  }
  const int k_eff = min(a.budget, len);
  __syncthreads();

  // ---- 2. threshold T = smallest distance whose cumulative count reaches
  // k_eff; quota = how many of the ties at T are kept.
  if (wave == 0) {
    uint32_t loc = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int d = 7 * lane + j;
      if (d < kBins) loc += s_tot[0][d] + s_tot[1][d];
    }
    const uint32_t inc = wave_inclusive_scan_u32(loc);
    const uint64_t ball = __ballot(inc >= (uint32_t)k_eff);
    const int first = __builtin_ffsll((long long)ball) - 1;  // exists: the total is len >= k_eff
    if (lane == first) {
      uint32_t cum = inc - loc;
      int T = 7 * lane;
      for (int j = 0; j < 7; ++j) {
        const int d = 7 * lane + j;
        const uint32_t nc = cum + s_tot[0][d] + s_tot[1][d];
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
  const uint32_t T = (uint32_t)s_T;
  const uint32_t quota = s_quota;
  const uint32_t biasT = (0x8000u - T) * 0x10001u;        // d >= T
  const uint32_t biasT1 = (0x8000u - T - 1u) * 0x10001u;  // d >= T + 1

  // ---- 3. ordered compaction.  Thread t owns positions [base + 64t, +64) of
  // a pass; every distance < T is kept, ties at T while the running tie count
  // (in position order) is below quota.  This split keeps global ranks
  // [lo_rank, hi_rank) of the selection.
  const int lo_rank = split * a.rows_per_split;
  const int hi_rank = min(lo_rank + a.rows_per_split, k_eff);
  uint32_t carry_eq = 0, carry_sel = 0;
#pragma unroll 1
  for (int base = 0; base < len && lo_rank < hi_rank && (int)carry_sel < hi_rank; base += kSAPass) {
    const int pos0 = base + tid * kSAPPT;
    if (base != 0) {
#pragma unroll
      for (int i = 0; i < kSAPPT / 8; ++i) dw[i] = drow[min((base >> 3) + tid * (kSAPPT / 8) + i, dmax16)];
    }
    if (pos0 + kSAPPT > len) {
#pragma unroll
      for (int i = 0; i < kSAPPT / 8; ++i) dw[i] = masked_dists(dw[i], pos0 + 8 * i, len);
    }
    uint32_t ge = 0, ge1 = 0;
#pragma unroll
    for (int i = 0; i < kSAPPT / 8; ++i) {
      ge += count_ge2(dw[i].x, biasT) + count_ge2(dw[i].y, biasT) + count_ge2(dw[i].z, biasT) +
            count_ge2(dw[i].w, biasT);
      ge1 += count_ge2(dw[i].x, biasT1) + count_ge2(dw[i].y, biasT1) + count_ge2(dw[i].z, biasT1) +
             count_ge2(dw[i].w, biasT1);
    }
    const uint32_t lt = kSAPPT - ge;  // masked positions count as >= T
    const uint32_t eq = ge - ge1;
    uint32_t tot_eq, tot_sel;
    const uint32_t e_before = carry_eq + block_exclusive_scan(eq, s_wsum, tot_eq);
    const uint32_t take = quota > e_before ? min(quota - e_before, eq) : 0u;
    const uint32_t s_before = carry_sel + block_exclusive_scan(lt + take, s_wsum, tot_sel);
    if (lt + take > 0 && (int)s_before < hi_rank && (int)(s_before + lt + take) > lo_rank) {
      uint32_t r = s_before, ties = 0;
#pragma unroll 1
      for (int i = 0; i < kSAPPT / 8; ++i) {
        uint4 w = drow[min((pos0 >> 3) + i, dmax16)];
        w = masked_dists(w, pos0 + 8 * i, len);
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t d = (ww[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
          bool keep = d < T;
          if (d == T) keep = ties++ < take;
          if (keep) {
            if ((int)r >= lo_rank && (int)r < hi_rank) {
              const int pp = pos0 + 8 * i + j;
              s_list[r - lo_rank] = pp;
              if (a.sel_idx) a.sel_idx[(size_t)bh * a.budget + r] = pp;
            }
            ++r;
          }
        }
      }
    }
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  if (a.sel_idx && split == 0) {
    for (int i = k_eff + tid; i < a.budget; i += kSAThreads) a.sel_idx[(size_t)bh * a.budget + i] = -1;
  }
  const int nrows = max(0, hi_rank - lo_rank);
  if (tid == 0) {
    s_m = -INFINITY;
    s_l = 0.f;
  }
  __syncthreads();

  // ---- 4. attention over the split's rows: tiles of 128 rows (16 per wave).
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;
  const uint16_t* Kg = a.k + ((size_t)b * a.Hkv + g) * (size_t)a.cap * kHeadDim;
  const uint16_t* Vg = a.v + ((size_t)b * a.Hkv + g) * (size_t)a.cap * kHeadDim;
#pragma unroll 1
  for (int t0 = 0; t0 < nrows; t0 += kSATile) {
    uint4 ka[4], vv[4];
    {
      const int ia = t0 + 16 * wave + col;
      const int pa = s_list[ia < nrows ? ia : 0];
      const uint16_t* kr = Kg + (size_t)pa * kHeadDim + 8 * kg;
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = *reinterpret_cast<const uint4*>(kr + 32 * s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int iv = t0 + 16 * wave + 4 * i + kg;
        const int pv = s_list[iv < nrows ? iv : 0];
        vv[i] = *reinterpret_cast<const uint4*>(Vg + (size_t)pv * kHeadDim + 8 * col);
      }
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_16x16x32_bf16(ka[s], qf[s], acc);
    if (col == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * wave + 4 * kg + i;
        s_S[rr] = t0 + rr < nrows ? acc[i] * a.qscale : -INFINITY;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const float x0 = s_S[lane], x1 = s_S[lane + 64];
      const float mo = s_m;
      const float mn = fmaxf(mo, wave_max(fmaxf(x0, x1)));  // finite: the tile has >= 1 row
      const float cr = exp2f(mo - mn);
      const float p0 = x0 == -INFINITY ? 0.f : exp2f(x0 - mn);
      const float p1 = x1 == -INFINITY ? 0.f : exp2f(x1 - mn);
      s_S[lane] = p0;
      s_S[lane + 64] = p1;
      const float ts = wave_sum(p0 + p1);
      if (lane == 0) {
        s_corr = cr;
        s_m = mn;
        s_l = __builtin_fmaf(s_l, cr, ts);
      }
    }
    __syncthreads();
    const float cr = s_corr;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] *= cr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pr = s_S[16 * wave + 4 * i + kg];
      const uint32_t vw[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        o[2 * j] = __builtin_fmaf(pr, bf16_lo(vw[j]), o[2 * j]);
        o[2 * j + 1] = __builtin_fmaf(pr, bf16_hi(vw[j]), o[2 * j + 1]);
      }
    }
    __syncthreads();
  }
  // reduce o over the four k-groups of each wave, then over the waves
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float v = o[j];
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    o[j] = v;
  }
  if (kg == 0) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_red[wave][8 * col + j] = o[j];
  }
  __syncthreads();

  if (a.splits == 1) {
    if (tid < kHeadDim) {
      float O = 0.f;
#pragma unroll
      for (int w = 0; w < kSAWaves; ++w) O += s_red[w][tid];
      a.out[(size_t)bh * kHeadDim + tid] = O / s_l;
    }
    return;
  }

  // ---- 5. several splits: publish (m, l, o) write-through, count, and let the
  // last split of this head merge them.
  float* pc = a.part + ((size_t)bh * a.splits + split) * kPartFloats;
  if (tid < kHeadDim) {
    float O = 0.f;
#pragma unroll
    for (int w = 0; w < kSAWaves; ++w) O += s_red[w][tid];
    store_coherent(pc + 4 + tid, O);
    if (tid == 0) {
      store_coherent(pc, s_m);
      store_coherent(pc + 1, s_l);
    }
  }
  wait_memory();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(a.splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (tid < kHeadDim) {
    const float* p0 = a.part + (size_t)bh * a.splits * kPartFloats;
    float M = -INFINITY;
#pragma unroll 1
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      float mv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) mv[u] = load_coherent(p0 + (size_t)min(s0 + u, a.splits - 1) * kPartFloats);
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, mv[u]);
    }
    float L = 0.f, O = 0.f;
#pragma unroll 1
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      float mv[8], lv[8], ov[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* ps = p0 + (size_t)min(s0 + u, a.splits - 1) * kPartFloats;
        mv[u] = load_coherent(ps);
        lv[u] = load_coherent(ps + 1);
        ov[u] = load_coherent(ps + 4 + tid);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < a.splits && mv[u] != -INFINITY) {
          const float wgt = exp2f(mv[u] - M);
          L = __builtin_fmaf(lv[u], wgt, L);
          O = __builtin_fmaf(ov[u], wgt, O);
        }
      }
    }
    a.out[(size_t)bh * kHeadDim + tid] = O / L;
  }
}

// --------------------------------------------------------------------------
// Launcher
// --------------------------------------------------------------------------

template <typename Kernel, typename... Args>
static void launch_k(int i, Kernel kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
  const ProfileEvents& pe = profile_events();
  if (2 * i + 1 < pe.n)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, pe.ev[2 * i], pe.ev[2 * i + 1], 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

template <int R>
static void launch_scan(const Plan& p, const ScanArgs& sa, hipStream_t s) {
  launch_k(0, scan_kernel<R>, dim3(p.nch, p.B * p.Hkv), dim3(kScanThreads), 0, s, sa);
}

hipError_t launch_decode(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* codes,
                         bool append, const int32_t* kv_len, float scale, float* out, int32_t* sel_idx,
                         uint16_t* dist, uint8_t* q_codes, char* ws, hipStream_t s) {
  uint16_t* ws_dist = reinterpret_cast<uint16_t*>(ws + p.off_dist);
  uint16_t* ws_hist = reinterpret_cast<uint16_t*>(ws + p.off_hist);
  float* ws_part = reinterpret_cast<float*>(ws + p.off_part);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + p.off_count);

  ScanArgs sa{q,        k,       codes,   kv_len, ws_dist, dist,    ws_hist, q_codes,
              counters, p.Hq,    p.Hkv,   p.cap,  p.dstride, p.chunk, p.nch, append ? 1 : 0};
  switch (p.R) {
    case 1: launch_scan<1>(p, sa, s); break;
    case 2: launch_scan<2>(p, sa, s); break;
    case 4: launch_scan<4>(p, sa, s); break;
    case 8: launch_scan<8>(p, sa, s); break;
    default: return hipErrorInvalidValue;
  }
  SelAttArgs aa{q,      k,        v,       kv_len, ws_dist, ws_hist, ws_part, counters, sel_idx, out,
                scale * 1.4426950408889634f, p.Hq, p.Hkv, p.R, p.cap, p.dstride, p.budget, p.chunk, p.nch,
                p.splits, p.rows_per_split};
  const size_t lds = (size_t)p.rows_per_split * sizeof(int);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&select_attend_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  launch_k(1, select_attend_kernel, dim3(p.B * p.Hq, p.splits), dim3(kSAThreads), (uint32_t)lds, s, aa);
  return hipGetLastError();
}

}  // namespace adamas
