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
// The same permute with no "old" operand (every lane is written), so that the
// compiler can fold it into the consuming add as a DPP source.
template <int CTRL>
__device__ __forceinline__ float quad_perm_src(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
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

// x[i] += s * (x[i] of the quad partner), i = base .. base+15, in one v_fmac_f32
// per element with the partner read through a quad_perm DPP source (the
// compiler does not fold a DPP move into fmac by itself).  A VALU write of a
// VGPR needs two wait states before a DPP read of it, and the hazard pass does
// not look inside asm: the block opens with s_nop 1, and inside it no
// instruction reads through DPP a register written earlier in the block.
#define ADAMAS_FMAC_DPP(i, sel) "v_fmac_f32_dpp %" #i ", %" #i ", %16 " sel " row_mask:0xf bank_mask:0xf\n"
#define ADAMAS_FMAC_DPP16(sel)                                                                              \
  "s_nop 1\n" ADAMAS_FMAC_DPP(0, sel) ADAMAS_FMAC_DPP(1, sel) ADAMAS_FMAC_DPP(2, sel) ADAMAS_FMAC_DPP(3, sel) \
      ADAMAS_FMAC_DPP(4, sel) ADAMAS_FMAC_DPP(5, sel) ADAMAS_FMAC_DPP(6, sel) ADAMAS_FMAC_DPP(7, sel)        \
      ADAMAS_FMAC_DPP(8, sel) ADAMAS_FMAC_DPP(9, sel) ADAMAS_FMAC_DPP(10, sel) ADAMAS_FMAC_DPP(11, sel)      \
      ADAMAS_FMAC_DPP(12, sel) ADAMAS_FMAC_DPP(13, sel) ADAMAS_FMAC_DPP(14, sel) ADAMAS_FMAC_DPP(15, sel)
template <int CTRL>
__device__ __forceinline__ void fmac_quad16(float (&x)[32], int base, float s) {
  static_assert(CTRL == kQuadXor1 || CTRL == kQuadXor2, "quad partner permutes only");
  float* y = x + base;
#define ADAMAS_FMAC_OPERANDS                                                                                   \
  : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), \
    "+v"(y[9]), "+v"(y[10]), "+v"(y[11]), "+v"(y[12]), "+v"(y[13]), "+v"(y[14]), "+v"(y[15])                   \
  : "v"(s)
  if constexpr (CTRL == kQuadXor1)
    asm(ADAMAS_FMAC_DPP16("quad_perm:[1,0,3,2]") ADAMAS_FMAC_OPERANDS);
  else
    asm(ADAMAS_FMAC_DPP16("quad_perm:[2,3,0,1]") ADAMAS_FMAC_OPERANDS);
#undef ADAMAS_FMAC_OPERANDS
}
#undef ADAMAS_FMAC_DPP16
#undef ADAMAS_FMAC_DPP

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
  // Half-widths 32 and 64 pair lane q with q ^ 1, then q ^ 2.  Each lane forms
  // own + s * partner in one fma with the partner as a DPP source: the lane with
  // the bit clear (s = +1) gets a + b; the lane with it set (s = -1) gets b - a,
  // the exact negation of the textbook a - b (products by +-1 are exact and
  // round-to-nearest is symmetric, so the fma rounds exactly like the add or
  // subtract it replaces).  A lane therefore holds sigma * y with
  // sigma = s32 * s64, i.e. -1 for quarters 1 and 2, +1 for quarters 0 and 3;
  // the sign of a zero never matters, since a zero only ever yields a zero.
  const float s32 = (quarter & 1) ? -1.0f : 1.0f;
  const float s64 = (quarter & 2) ? -1.0f : 1.0f;
  fmac_quad16<kQuadXor1>(x, 0, s32);
  fmac_quad16<kQuadXor1>(x, 16, s32);
  fmac_quad16<kQuadXor2>(x, 0, s64);
  fmac_quad16<kQuadXor2>(x, 16, s64);
  const float sigma = s32 * s64;
  // m = max |y| over the 128 coordinates (exact), t = m / 2
  float m = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) m = fmaxf(m, fabsf(x[e]));
  m = fmaxf(m, quad_perm_src<kQuadXor1>(m));
  m = fmaxf(m, quad_perm_src<kQuadXor2>(m));
  const float t = 0.5f * m;
  // code = [y >= -t] + [y >= 0] + [y >= t]; high bit = [y >= 0], low bit = 1 for
  // codes 1 and 3.  With y = sigma * held + 0 (exact, and -0 maps to +0 so that
  // -0 counts as "not below 0"): for y >= 0 the low bit is [y >= t], for y < 0
  // it is [y >= -t]; both are "y - copysign(t, y) is not below 0", read from the
  // sign bit of that exactly-signed difference (an exact zero is +0).  The
  // negated sign bits are shifted into the two words, coordinate 31 first.
  uint32_t nlo = 0, nhi = 0;
#pragma unroll
  for (int e = 31; e >= 0; --e) {
    const float y = __builtin_fmaf(x[e], sigma, 0.0f);
    const float v = y - __builtin_copysignf(t, y);
    nlo = __builtin_amdgcn_alignbit(nlo, __float_as_uint(v), 31);
    nhi = __builtin_amdgcn_alignbit(nhi, __float_as_uint(y), 31);
  }
  lo_word = ~nlo;
  hi_word = ~nhi;
}

// ---- wave-wide reductions (64 lanes) with DPP inside each 16-lane row and
// readlane across the four rows; the result is wave-uniform.
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kQuadXor1>(v);
  v += dpp_f<kQuadXor2>(v);
  v += dpp_f<kDppRowHalfMirror>(v);
  v += dpp_f<kDppRowMirror>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kQuadXor1>(v));
  v = fmaxf(v, dpp_f<kQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppRowMirror>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u<kQuadXor1>(v);
  v += dpp_u<kQuadXor2>(v);
  v += dpp_u<kDppRowHalfMirror>(v);
  v += dpp_u<kDppRowMirror>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Inclusive prefix sum over the 64 lanes of a wave (DPP: shifts within each
// 16-lane row, then row broadcasts of lanes 15 and 31).
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ uint32_t wave_inclusive_scan_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr1, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr2, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr4, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowShr8, 0xF, 0xF, true);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false);
  return v;
}

// Largest value over the 64 lanes (unsigned): maxima inside each 16-lane row,
// then row broadcasts carry rows 0-2 into row 3; lane 63 holds the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<kQuadXor1>(v));
  v = max(v, dpp_u<kQuadXor2>(v));
  v = max(v, dpp_u<kDppRowHalfMirror>(v));
  v = max(v, dpp_u<kDppRowMirror>(v));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast15, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// The value held by lane (lane ^ X), X = 1, 2, 3, 4, 7, 8, 15, 16, 31 or 63,
// without the LDS crossbar: DPP row permutes inside 16-lane rows (xor 4 as a
// shift left or right by 4, whichever stays inside the lane's group of 8), the
// gfx950 lane-swap instructions across rows (v_permlane16_swap exchanges lanes
// l and l ^ 16, v_permlane32_swap lanes l and l ^ 32), and compositions of
// these (xor 31 = xor 16 of xor 15, xor 63 = xor 32 of xor 31).
constexpr int kQuadMirror = 0x1B;   // quad_perm [3,2,1,0] = xor 3
constexpr int kDppRowRor8 = 0x128;  // rotate by 8 inside a 16-lane row = xor 8
constexpr int kDppRowShl4 = 0x104;  // lane l takes lane l + 4 (inside the row)

__device__ __forceinline__ uint32_t xor16_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // {rows 1,3 <- rows 0,2; rows 0,2 <- rows 1,3}
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // {lanes 32.. <- 0..; lanes 0.. <- 32..}
  return (threadIdx.x & 32) ? r[0] : r[1];
}
template <int X>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t v) {
  if constexpr (X == 1) return dpp_u<kQuadXor1>(v);
  else if constexpr (X == 2) return dpp_u<kQuadXor2>(v);
  else if constexpr (X == 3) return dpp_u<kQuadMirror>(v);
  else if constexpr (X == 4) {
    // (both shifts with every lane active, then a branch-free pick: a
    // conditional expression here becomes a branch, and a DPP read from a
    // lane outside the branch returns nothing)
    const uint32_t from_below = dpp_u<kDppRowShr4>(v), from_above = dpp_u<kDppRowShl4>(v);
    const uint32_t pick = 0u - ((threadIdx.x >> 2) & 1u);
    return from_above ^ ((from_below ^ from_above) & pick);
  }
  else if constexpr (X == 7) return dpp_u<kDppRowHalfMirror>(v);
  else if constexpr (X == 8) return dpp_u<kDppRowRor8>(v);
  else if constexpr (X == 15) return dpp_u<kDppRowMirror>(v);
  else if constexpr (X == 16) return xor16_u32(v);
  else if constexpr (X == 31) return xor16_u32(dpp_u<kDppRowMirror>(v));
  else return xor32_u32(xor16_u32(dpp_u<kDppRowMirror>(v)));  // X == 63
}

// One compare-exchange step: the lower lane of each pair keeps the minimum.
template <int X>
__device__ __forceinline__ uint32_t cmp_xchg(uint32_t key, int lane, int low_bit) {
  const uint32_t other = lane_xor_u32<X>(key);
  return (lane & low_bit) == 0 ? min(key, other) : max(key, other);
}

// Ascending sort of one key per lane inside every aligned group of S lanes (S a
// power of two, 1..64): bitonic sort in the form where stage k first compares
// lane i with its mirror i ^ (k-1) inside the k-block, then half-cleans with
// i ^ j for j = k/4, ..., 1, every comparison ascending.  All lanes active.
template <int K>
__device__ __forceinline__ uint32_t sort_stage(uint32_t key, int lane) {
  key = cmp_xchg<K - 1>(key, lane, K >> 1);
  if constexpr (K >= 64) key = cmp_xchg<16>(key, lane, 16);
  if constexpr (K >= 32) key = cmp_xchg<8>(key, lane, 8);
  if constexpr (K >= 16) key = cmp_xchg<4>(key, lane, 4);
  if constexpr (K >= 8) key = cmp_xchg<2>(key, lane, 2);
  if constexpr (K >= 4) key = cmp_xchg<1>(key, lane, 1);
  return key;
}
template <int S>
__device__ __forceinline__ uint32_t group_sort_u32(uint32_t key) {
  const int lane = (int)(threadIdx.x & 63);
  if constexpr (S >= 2) key = sort_stage<2>(key, lane);
  if constexpr (S >= 4) key = sort_stage<4>(key, lane);
  if constexpr (S >= 8) key = sort_stage<8>(key, lane);
  if constexpr (S >= 16) key = sort_stage<16>(key, lane);
  if constexpr (S >= 32) key = sort_stage<32>(key, lane);
  if constexpr (S >= 64) key = sort_stage<64>(key, lane);
  return key;
}

// ---- coherent global accesses between blocks of one kernel.  A store at agent
// scope writes through the XCD's L2 and an agent-scope load bypasses it, so a
// block can publish results to a later block on another XCD without flushing
// the whole L2 (which a device-scope fence does on this chip).
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte and 2-byte accesses of data handed between blocks of one kernel:
// written through (agent-scope atomic stores) and read coherently
// (agent-scope atomic loads), so that the reader sees the writer's data
// whatever XCD either runs on.  kCoherent = false: plain accesses (data that
// a kernel boundary hands over).
template <bool kCoherent>
__device__ __forceinline__ void st16(void* p, uint4 v) {
  if constexpr (kCoherent) {
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<uint4*>(p) = v;
  }
}
template <bool kCoherent>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (kCoherent) {
    const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
    const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_uint4((uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32));
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}
// A raw buffer resource (stride 0) over the n bytes at p: a buffer load at a
// byte offset >= n returns 0 and reads no memory.  Word 3 holds the untyped
// 32-bit data format of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 as_uint4(__attribute__((ext_vector_type(4))) unsigned int v) {
  return make_uint4(v[0], v[1], v[2], v[3]);
}
template <bool kCoherent>
__device__ __forceinline__ uint32_t ld_u16(const uint16_t* p) {
  if constexpr (kCoherent) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t w = __hip_atomic_load(reinterpret_cast<const uint32_t*>(a & ~(uintptr_t)3), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return (a & 2) ? (w >> 16) : (w & 0xFFFFu);
  } else {
    return *p;
  }
}
// The same for a rare global read beside an LDS read of the same variable:
// the plain form is volatile, so that the two are never merged into one
// generic (flat) load with a full wait.
template <bool kCoherent>
__device__ __forceinline__ uint32_t ld_u16_apart(const uint16_t* p) {
  if constexpr (kCoherent) return ld_u16<true>(p);
  else return *reinterpret_cast<const volatile uint16_t*>(p);
}

// Wait until every memory operation this thread issued has completed (for the
// write-through stores above: reached the point of coherence).  The signal
// fence keeps the compiler from moving the stores past the wait.
__device__ __forceinline__ void wait_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- MFMA 16x16x32 bf16 (gfx950).  Operand layout, lane l = 0..63:
//   A (16 x 32): lane holds A[l % 16][8 * (l / 16) .. +8]
//   B (32 x 16): lane holds B[8 * (l / 16) .. +8][l % 16]
//   C (16 x 16): lane holds C[4 * (l / 16) + i][l % 16], i = 0..3
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// (readfirstlane: tells the compiler the value is the same in every lane of
// the wave, so loops and branches on it stay scalar)
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Number of set bits of `mask` in lanes below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace adamas
