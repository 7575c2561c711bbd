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
//                      one (m, l, o) partial per head
// combine_kernel       per (b, kv head): merges the chunk partials into out
// (The sparse decode step itself lives in decode.hip.)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "plan.h"

namespace adamas {

// --------------------------------------------------------------------------
// Key encode
// --------------------------------------------------------------------------

// grid (nblk, B*Hkv), 256 threads = 64 vectors per pass (a quad per vector).
template <bool kPaged>
__global__ __launch_bounds__(256) void encode_keys_kernel(const uint16_t* __restrict__ k,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ end,
                                                          uint8_t* __restrict__ codes, KvLayout kv) {
  const int bg = blockIdx.y;
  const int b = bg / kv.Hkv;
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
  float qscale;         // softmax scale * log2(e)
  int Hq, Hkv, cap, chunk, nch;
  KvLayout kv;
};

// Merge the per-chunk partials (m, l, o[128]) of R heads into out.  `part`
// points at head 0's partials; head r's are r * nch chunks further.  Runs with
// all threads of the block.  Loads are issued in batches with clamped indices
// so that they overlap.
template <int R>
__device__ __forceinline__ void combine_group(const float* __restrict__ part, int nch, int nch_b,
                                              float* __restrict__ out, float (*s_w)[kMaxChunks], float* s_L) {
  auto ld = [](const float* p) { return *p; };
  const int tid = threadIdx.x;
  // 1. m and l of every (head, chunk)
  for (int i = tid; i < R * kMaxChunks; i += 256) {
    const int r = i / kMaxChunks, c = i - r * kMaxChunks;
    const float* pc = part + ((size_t)r * nch + (c < nch_b ? c : 0)) * kPartFloats;
    const float m = ld(pc);
    const float l = ld(pc + 1);
    s_w[r][c] = c < nch_b ? m : -INFINITY;
    if (c < nch_b) s_L[R + r * kMaxChunks + c] = l;  // scratch: l values after the R totals
  }
  __syncthreads();
  // 2. per head: M = max m, weights 2^(m - M), L = sum weight * l
  for (int r = wave_id(); r < R; r += 4) {
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
  // 3. out[r][d] = sum_c w_c o_c[d] / L, 16 loads in flight per thread
  for (int i = tid; i < R * kHeadDim; i += 256) {
    const int r = i / kHeadDim, d = i - r * kHeadDim;
    const float* pr = part + (size_t)r * nch * kPartFloats + 4 + d;
    float O = 0.f;
    for (int c0 = 0; c0 < nch_b; c0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = ld(pr + (size_t)min(c0 + u, nch_b - 1) * kPartFloats);
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + u < nch_b) O = __builtin_fmaf(s_w[r][c0 + u], v[u], O);
    }
    out[(size_t)r * kHeadDim + d] = O / s_L[r];
  }
}

template <int R>
struct AttnSmem {
  float S[64][R + 1];     // scores, then probabilities, of one 64-row tile
  float mrun[R], lrun[R], corr[R];
  float red[4][R][kHeadDim];
};

// Exact softmax attention of the group's R queries over positions
// [p0, p0 + nrows) of one KV head, written as one partial (m, l, o[128]) per
// head: m = running max of the scaled log2 scores, l = sum 2^(s - m),
// o = sum 2^(s - m) V.
//   q . K^T: MFMA 16x16x32 bf16, 16 rows x 16 columns (the R heads, rest zero)
//            per wave, 64 rows per tile;
//   P . V:   VALU, 16 lanes per row (8 dims each), 4 rows per instruction.
template <int R, bool kPaged>
__device__ __forceinline__ void attend_rows(const AttendArgs& a, int b, int g, int c, int p0, int nrows,
                                            AttnSmem<R>& sm) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int col = lane & 15;  // MFMA column = head (A: row in tile, PV: 8-dim block)
  const int kg = lane >> 4;   // MFMA k-group
  auto pos = [&](int i) { return p0 + i; };

  uint4 qf[4];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)(g * R + (col < R ? col : 0))) * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = col < R ? *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * kg) : make_uint4(0, 0, 0, 0);
  }
  if (tid < R) {
    sm.mrun[tid] = -INFINITY;
    sm.lrun[tid] = 0.f;
  }
  float o[R][8];
#pragma unroll
  for (int h = 0; h < R; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[h][j] = 0.f;
  // K and V rows of position p: Kg + kvoff(p), Vg + kvoff(p)
  const size_t kv_base = kPaged ? (size_t)0 : ((size_t)b * a.Hkv + g) * (size_t)a.cap * kHeadDim;
  const uint16_t* Kg = a.k + kv_base;
  const uint16_t* Vg = a.v + kv_base;
  auto kvoff = [&](int p) -> size_t {
    if constexpr (kPaged) return kv_row<true>(a.kv, b, g, p) * kHeadDim;
    else return (size_t)p * kHeadDim;
  };
  __syncthreads();

  for (int t0 = 0; t0 < nrows; t0 += 64) {
    // K rows for the A operand and V rows for P.V of this wave's 16 rows;
    // rows past the end are clamped to row 0 and masked out below.
    uint4 ka[4], vv[4];
    {
      const int ia = t0 + 16 * w + col;
      const int pa = pos(ia < nrows ? ia : 0);
      const uint16_t* kr = Kg + kvoff(pa) + 8 * kg;
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = *reinterpret_cast<const uint4*>(kr + 32 * s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int iv = t0 + 16 * w + 4 * i + kg;
        const int pv = pos(iv < nrows ? iv : 0);
        vv[i] = *reinterpret_cast<const uint4*>(Vg + kvoff(pv) + 8 * col);
      }
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_16x16x32_bf16(ka[s], qf[s], acc);
    if (col < R) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * w + 4 * kg + i;
        const int idx = t0 + rr;
        sm.S[rr][col] = idx < nrows ? acc[i] * a.qscale : -INFINITY;
      }
    }
    __syncthreads();
    // running max / rescale / probabilities: wave w owns heads w, w+4; lane = row
#pragma unroll
    for (int h = w; h < R; h += 4) {
      const float x = sm.S[lane][h];
      const float mo = sm.mrun[h];
      const float mn = fmaxf(mo, wave_max(x));
      const float cr = (mn == -INFINITY) ? 1.f : exp2f(mo - mn);
      const float pr = (x == -INFINITY) ? 0.f : exp2f(x - mn);
      sm.S[lane][h] = pr;
      const float ts = wave_sum(pr);
      if (lane == 0) {
        sm.corr[h] = cr;
        sm.mrun[h] = mn;
        sm.lrun[h] = __builtin_fmaf(sm.lrun[h], cr, ts);
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float cr = sm.corr[h];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[h][j] *= cr;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 16 * w + 4 * i + kg;
      const uint32_t vw[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vf[2 * j] = bf16_lo(vw[j]);
        vf[2 * j + 1] = bf16_hi(vw[j]);
      }
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const float pr = sm.S[rr][h];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[h][j] = __builtin_fmaf(pr, vf[j], o[h][j]);
      }
    }
    __syncthreads();
  }

  // reduce o over the four k-groups of the wave, then over the four waves
#pragma unroll
  for (int h = 0; h < R; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v = o[h][j];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      o[h][j] = v;
    }
  if (kg == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) sm.red[w][h][8 * col + j] = o[h][j];
  }
  __syncthreads();
  for (int i = tid; i < R * kHeadDim; i += 256) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    const float O = (sm.red[0][h][d] + sm.red[1][h][d]) + (sm.red[2][h][d] + sm.red[3][h][d]);
    float* pc = a.ws_part + (((size_t)b * a.Hq + (size_t)(g * R + h)) * a.nch + c) * kPartFloats;
    if (d == 0) {
      pc[0] = sm.mrun[h];
      pc[1] = sm.lrun[h];
    }
    pc[4 + d] = O;
  }
}

// Dense decode attention: block (c, b*Hkv + g) attends the group's R queries
// over positions [c*chunk, min((c+1)*chunk, kv_len[b])) and writes one partial
// per head; combine_kernel merges the chunks.
template <int R, bool kPaged>
__global__ __launch_bounds__(256) void dense_attend_kernel(AttendArgs a) {
  const int bg = blockIdx.y;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int c = blockIdx.x;
  const int len = min(a.kv_len[b], a.cap);  // (kv_len <= capacity is a precondition; clamped all the same)
  const int nch_b = (max(len, 0) + a.chunk - 1) / a.chunk;
  if (c >= nch_b) return;
  const int p0 = c * a.chunk;
  const int p1 = min(p0 + a.chunk, len);
  __shared__ AttnSmem<R> sm;
  attend_rows<R, kPaged>(a, b, g, c, p0, p1 - p0, sm);
}

// Dense path: one block per (b, kv head) merges the chunk partials of its R heads.
template <int R>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part, const int32_t* kv_len,
                                                      float* __restrict__ out, int Hq, int Hkv, int chunk,
                                                      int nch) {
  __shared__ float s_w[R][kMaxChunks];
  __shared__ float s_l[R * (kMaxChunks + 1)];
  const int bg = blockIdx.x;
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  // (clamped like the attend kernel's: the nch chunks cover the capacity)
  const int nch_b = (max(min(kv_len[b], nch * chunk), 0) + chunk - 1) / chunk;
  const size_t bh0 = (size_t)b * Hq + (size_t)(g * R);
  if (nch_b == 0) {  // no cached position: attention over the empty set is the zero vector
    for (int i = threadIdx.x; i < R * kHeadDim; i += 256) out[bh0 * kHeadDim + i] = 0.f;
    return;
  }
  combine_group<R>(part + bh0 * nch * kPartFloats, nch, nch_b, out + bh0 * kHeadDim, s_w, s_l);
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
                              const int32_t* end, uint8_t* codes, hipStream_t s) {
  const int bg = B * kv.Hkv;
  int nblk = (kv.cap + 63) / 64;
  const int cap_blocks = 2048 / bg > 0 ? 2048 / bg : 1;
  if (nblk > cap_blocks) nblk = cap_blocks;
  if (kv.table)
    launch_k(0, encode_keys_kernel<true>, dim3(nblk, bg), dim3(256), 0, s, k, start, end, codes, kv);
  else
    launch_k(0, encode_keys_kernel<false>, dim3(nblk, bg), dim3(256), 0, s, k, start, end, codes, kv);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_dense_r(const Plan& p, const KvLayout& kv, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const int32_t* kv_len, float scale, float* out, char* ws,
                                 hipStream_t s) {
  float* ws_part = reinterpret_cast<float*>(ws + p.off_part);
  AttendArgs aa{q, k, v, kv_len, ws_part, scale * 1.4426950408889634f, p.Hq, p.Hkv, p.cap, p.chunk, p.nch, kv};
  if (kv.table)
    launch_k(0, dense_attend_kernel<R, true>, dim3(p.nch, p.B * p.Hkv), dim3(256), 0, s, aa);
  else
    launch_k(0, dense_attend_kernel<R, false>, dim3(p.nch, p.B * p.Hkv), dim3(256), 0, s, aa);
  if (profile_events().n >= 4) {  // timing mode: see adamas_profile_events
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
  }
  launch_k(1, combine_kernel<R>, dim3(p.B * p.Hkv), dim3(256), 0, s, (const float*)ws_part, kv_len, out, p.Hq,
           p.Hkv, p.chunk, p.nch);
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
