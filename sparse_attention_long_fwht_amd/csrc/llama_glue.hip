// llama_glue.hip -- the per-layer elementwise work of a Llama-shaped decode
// step between its GEMMs, fused into three kernels (libllama_glue.so, declared
// in include/llama_glue.h).  Not part of the Adamas method: these are the model
// around the decode step, used to measure it end to end against dense attention
// (paper abstracts and blog section 5.1: end-to-end speedup on
// Llama-3.1-8B-Instruct).  Unfused, this work is some thirty tiny launches per
// layer, which would dominate a one-token decode step.
//
// All tensors bf16 (raw 16-bit storage) unless noted; arithmetic in fp32, one
// rounding to bf16 per stored value.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "llama_glue.h"

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t to_bf(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float block_sum(float v, float* s_red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += s_red[w];
  return t;
}

// x_out = x + delta (bf16), h = bf16(x_out * rsqrt(mean(x_out^2) + eps) * w).
// One block per row; H % 8 == 0, H <= 8 * kThreads * 8.
__global__ __launch_bounds__(kThreads) void add_rmsnorm_kernel(const uint16_t* x, const uint16_t* delta,
                                                               uint16_t* x_out, const uint16_t* w, uint16_t* h,
                                                               int H, float eps) {
  __shared__ float s_red[kThreads / 64];
  const size_t row = (size_t)blockIdx.x * H;
  constexpr int kMaxPer = 8;  // 8-element groups per thread
  float v[kMaxPer][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = (i * kThreads + (int)threadIdx.x) * 8;
    if (c < H) {
      const uint4 a = *reinterpret_cast<const uint4*>(x + row + c);
      const uint16_t* ah = reinterpret_cast<const uint16_t*>(&a);
      uint4 d = make_uint4(0u, 0u, 0u, 0u);
      if (delta) d = *reinterpret_cast<const uint4*>(delta + row + c);
      const uint16_t* dh = reinterpret_cast<const uint16_t*>(&d);
      uint16_t o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        o[j] = delta ? to_bf(bf(ah[j]) + bf(dh[j])) : ah[j];
        v[i][j] = bf(o[j]);
        ss += v[i][j] * v[i][j];
      }
      if (x_out) *reinterpret_cast<uint4*>(x_out + row + c) = *reinterpret_cast<const uint4*>(o);
    }
  }
  const float r = rsqrtf(block_sum(ss, s_red) / (float)H + eps);
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int c = (i * kThreads + (int)threadIdx.x) * 8;
    if (c < H) {
      const uint4 ww = *reinterpret_cast<const uint4*>(w + c);
      const uint16_t* wh = reinterpret_cast<const uint16_t*>(&ww);
      uint16_t o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = to_bf(v[i][j] * r * bf(wh[j]));
      *reinterpret_cast<uint4*>(h + row + c) = *reinterpret_cast<const uint4*>(o);
    }
  }
}

// Rotary embedding (halves rotated: element i pairs with i + 64) of the query
// and key heads of one token, at position pos[b]; writes q (contiguous) and the
// key and value rows into the caches at that position.  Block b, thread t:
// pair (head t / 64, element t % 64) of the Hq + Hkv rotated heads, then the
// value copy.
__global__ __launch_bounds__(kThreads) void rope_append_kernel(const uint16_t* qkv, const int32_t* pos,
                                                               const float* inv_freq, uint16_t* q_out,
                                                               uint16_t* k_cache, uint16_t* v_cache, int Hq,
                                                               int Hkv, int cap) {
  const int b = blockIdx.x;
  const int p = pos[b];
  // a position outside the cache (a precondition violated) writes no cache row
  const bool in_cache = p >= 0 && p < cap;
  const int width = (Hq + 2 * Hkv) * 128;
  const uint16_t* src = qkv + (size_t)b * width;
  for (int t = threadIdx.x; t < (Hq + Hkv) * 64; t += kThreads) {
    const int hh = t >> 6, i = t & 63;
    if (hh >= Hq && !in_cache) break;  // (heads in order: only cache rows follow)
    const float ang = (float)p * inv_freq[i];
    const float c = cosf(ang), s = sinf(ang);
    const float x1 = bf(src[hh * 128 + i]), x2 = bf(src[hh * 128 + 64 + i]);
    const uint16_t y1 = to_bf(x1 * c - x2 * s), y2 = to_bf(x2 * c + x1 * s);
    uint16_t* dst = hh < Hq ? q_out + ((size_t)b * Hq + hh) * 128
                            : k_cache + (((size_t)b * Hkv + (hh - Hq)) * cap + p) * 128;
    dst[i] = y1;
    dst[64 + i] = y2;
  }
  if (!in_cache) return;
  for (int t = threadIdx.x; t < Hkv * 128; t += kThreads) {
    const int g = t >> 7, i = t & 127;
    v_cache[(((size_t)b * Hkv + g) * cap + p) * 128 + i] = src[(Hq + Hkv) * 128 + t];
  }
}

// out[b][i] = bf16(silu(gate) * up), gate = gu[b][i], up = gu[b][F + i].
__global__ __launch_bounds__(kThreads) void silu_mul_kernel(const uint16_t* gu, uint16_t* out, int F) {
  const int b = blockIdx.y;
  const int i = (blockIdx.x * kThreads + threadIdx.x) * 8;
  if (i >= F) return;
  const uint4 g4 = *reinterpret_cast<const uint4*>(gu + (size_t)b * 2 * F + i);
  const uint4 u4 = *reinterpret_cast<const uint4*>(gu + (size_t)b * 2 * F + F + i);
  const uint16_t* gh = reinterpret_cast<const uint16_t*>(&g4);
  const uint16_t* uh = reinterpret_cast<const uint16_t*>(&u4);
  uint16_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float g = bf(gh[j]);
    o[j] = to_bf(g / (1.f + expf(-g)) * bf(uh[j]));
  }
  *reinterpret_cast<uint4*>(out + (size_t)b * F + i) = *reinterpret_cast<const uint4*>(o);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

int32_t llama_add_rmsnorm(const void* x, const void* delta, void* x_out, const void* w, void* h, int32_t rows,
                          int32_t hidden, float eps, void* stream) {
  if (!x || !w || !h || rows < 1 || hidden < 8 || hidden % 8 != 0) return 1;
  if (hidden > 8 * kThreads * 8) return 2;
  if (!aligned16(x) || !aligned16(w) || !aligned16(h) || (delta && !aligned16(delta)) ||
      (x_out && !aligned16(x_out)))
    return 1;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(rows), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(delta),
                     static_cast<uint16_t*>(x_out), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(h),
                     hidden, eps);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t llama_rope_append(const void* qkv, const int32_t* pos, const float* inv_freq, void* q_out, void* k_cache,
                          void* v_cache, int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t capacity,
                          void* stream) {
  if (!qkv || !pos || !inv_freq || !q_out || !k_cache || !v_cache || batch < 1 || q_heads < 1 || kv_heads < 1 ||
      capacity < 1)
    return 1;
  hipLaunchKernelGGL(rope_append_kernel, dim3(batch), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(qkv), pos, inv_freq, static_cast<uint16_t*>(q_out),
                     static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), q_heads, kv_heads, capacity);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int32_t llama_silu_mul(const void* gu, void* out, int32_t rows, int32_t ffn, void* stream) {
  if (!gu || !out || rows < 1 || ffn < 8 || ffn % 8 != 0) return 1;
  if (!aligned16(gu) || !aligned16(out)) return 1;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((ffn / 8 + kThreads - 1) / kThreads, rows), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(gu),
                     static_cast<uint16_t*>(out), ffn);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
