// device_common.h -- gfx950 device helpers shared by the Adamas kernels.
//
// Encoding of one 128-dim head vector (sources: "Adamas: Hadamard Sparse
// Attention for Efficient Long-Context Inference", v1/v2 abstracts -- transform,
// bucketize, 2-bit compress; "ADAMAS：稀疏注意力优化技术解析与应用实践" blog,
// section 2.1 -- O(n log n) transform, section 2.2 -- thresholds -t, 0, +t with
// t = max|y| / 2 and strict "<" tests).
//
// Lane layout: four lanes of a quad own one vector; lane j of the quad holds
// coordinates 32j .. 32j+31 in registers.  The butterflies of half-width 1..16
// run inside a lane, 32 and 64 across the quad with DPP quad permutes, in the
// order 1, 2, 4, ..., 64.  Every butterfly output is a single fp32 add or subtract
// of the same two operands as in the textbook stage-by-stage transform, so the
// result is bit-identical to it (an fma with a +-1 multiplier rounds once, like
// the add/sub it replaces).  No reassociation: this header is compiled with
// -ffp-contract=off and no fast-math.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace adamas {


// quad_perm DPP controls: lane i of each quad reads lane perm[i].
constexpr int kQuadXor1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // [2,3,0,1]

template <int CTRL>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Widen 32 bf16 values (four 16-byte words, little-endian pairs) to fp32 exactly.
__device__ __forceinline__ void widen32(const uint4 (&w)[4], float (&x)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[8 * i + 0] = bf16_lo(w[i].x);
    x[8 * i + 1] = bf16_hi(w[i].x);
    x[8 * i + 2] = bf16_lo(w[i].y);
    x[8 * i + 3] = bf16_hi(w[i].y);
    x[8 * i + 4] = bf16_lo(w[i].z);
    x[8 * i + 5] = bf16_hi(w[i].z);
    x[8 * i + 6] = bf16_lo(w[i].w);
    x[8 * i + 7] = bf16_hi(w[i].w);
  }
}

// Transform, bucketize and pack one vector held by a quad (see the layout above).
// `quarter` = lane & 3.  Outputs this lane's 32 low-plane bits (code bit 0 of
// coordinates 32*quarter + e at bit e) and 32 high-plane bits.
__device__ __forceinline__ void encode_quad(float (&x)[32], int quarter, uint32_t& lo_word,
                                            uint32_t& hi_word) {
  // butterflies inside the lane: half-width 1, 2, 4, 8, 16
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if ((e & h) == 0) {
        const float a = x[e];
        const float b = x[e + h];
        x[e] = a + b;
        x[e + h] = a - b;
      }
    }
  }
  // half-width 32: partner is lane ^ 1.  The lane holding x[j] (bit clear) forms
  // own + partner; the lane holding x[j+32] forms partner - own.
  {
    const float sgn = (quarter & 1) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = __builtin_fmaf(x[e], sgn, quad_swap<kQuadXor1>(x[e]));
  }
  // half-width 64: partner is lane ^ 2
  {
    const float sgn = (quarter & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = __builtin_fmaf(x[e], sgn, quad_swap<kQuadXor2>(x[e]));
  }
  // m = max |y| over the 128 coordinates (exact), t = m / 2
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(x[e]));
  m = fmaxf(m, quad_swap<kQuadXor1>(m));
  m = fmaxf(m, quad_swap<kQuadXor2>(m));
  const float t = 0.5f * m;
  // code = [y >= -t] + [y >= 0] + [y >= t]; low bit = XOR of the three tests,
  // high bit = [y >= 0].  Each test is the sign bit of an exactly-signed value:
  // y + t < 0 iff y < -t, y < 0, y - t < 0 iff y < t, where y is first mapped
  // -0 -> +0 so that -0 counts as "not below 0" (and, with t = 0, not below t).
  // The sign bits (negated) are shifted into the two words, coordinate 31 first.
  uint32_t nlo = 0, nhi = 0;
#pragma unroll
  for (int e = 31; e >= 0; --e) {
    const float y = x[e] + 0.0f;
    const uint32_t sy = __float_as_uint(y);
    const uint32_t sl = __float_as_uint(y + t) ^ sy ^ __float_as_uint(y - t);
    nlo = __builtin_amdgcn_alignbit(nlo, sl, 31);
    nhi = __builtin_amdgcn_alignbit(nhi, sy, 31);
  }
  lo_word = ~nlo;
  hi_word = ~nhi;
}

// Wave-wide (64-lane) sum, result in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of `mask` in lanes below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace adamas
