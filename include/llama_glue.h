/*
 * llama_glue.h -- C ABI of libllama_glue.so (gfx950): the elementwise work of a
 * Llama-shaped decode step between its GEMMs, fused into three kernels.
 *
 * Not part of the Adamas method.  The pages measure Adamas end to end on
 * Llama-3.1-8B-Instruct ("Adamas: Hadamard Sparse Attention for Efficient
 * Long-Context Inference", v1/v2 abstracts: 1.5x end-to-end at 32K; the ADAMAS
 * blog, section 5.1: the same, memory bandwidth being the limit at 32K); these
 * kernels let a one-token decode step of that shape run without the dozens of
 * tiny launches per layer that plain tensor operations would take, so that the
 * end-to-end comparison measures the attention and the weights, not launch gaps.
 *
 * Conventions: bf16 tensors are raw 16-bit storage; pointers are caller-owned
 * device pointers to contiguous row-major memory, 16-byte aligned where noted;
 * `stream` is a hipStream_t (NULL = null stream); calls only enqueue work.
 * Arithmetic is fp32 with one round-to-nearest-even to bf16 per stored value.
 * Return: 0 ok, 1 invalid argument (nothing enqueued), 2 unsupported size,
 * 4 launch failure.
 */
#ifndef LLAMA_GLUE_H
#define LLAMA_GLUE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Residual add and RMSNorm of `rows` rows of `hidden` values:
 *   x_out = x + delta                      (delta NULL: x_out = x; x_out NULL: not stored;
 *                                           x_out may equal x)
 *   h     = (x_out / sqrt(mean(x_out^2) + eps)) * w
 * x, delta, x_out, h: bf16 [rows][hidden]; w: bf16 [hidden].  hidden % 8 == 0,
 * hidden <= 16384 (else 2); every pointer 16-byte aligned.
 */
int32_t llama_add_rmsnorm(const void* x, const void* delta, void* x_out, const void* w, void* h, int32_t rows,
                          int32_t hidden, float eps, void* stream);

/*
 * Rotary embedding and cache append for one new token per sequence.  qkv is the
 * fused projection, bf16 [batch][(q_heads + 2 kv_heads) * 128]: q heads, then k
 * heads, then v heads.  With a = pos[b] * inv_freq[i] (fp32), element i < 64 of
 * each q and k head pairs with element i + 64:
 *   y[i] = x[i] cos a - x[i+64] sin a,  y[i+64] = x[i+64] cos a + x[i] sin a.
 * Writes q_out bf16 [batch][q_heads][128], and row pos[b] of k_cache (rotated)
 * and v_cache (copied), both bf16 [batch][kv_heads][capacity][128].
 *   pos       int32 [batch] device; precondition 0 <= pos[b] < capacity (a
 *             position outside [0, capacity) writes q_out but no cache row)
 *   inv_freq  fp32 [64] device
 */
int32_t llama_rope_append(const void* qkv, const int32_t* pos, const float* inv_freq, void* q_out, void* k_cache,
                          void* v_cache, int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t capacity,
                          void* stream);

/*
 * SwiGLU gate: out[r][i] = silu(gu[r][i]) * gu[r][ffn + i], silu(g) = g / (1 + e^-g).
 * gu bf16 [rows][2 ffn], out bf16 [rows][ffn]; ffn % 8 == 0; 16-byte aligned.
 */
int32_t llama_silu_mul(const void* gu, void* out, int32_t rows, int32_t ffn, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_GLUE_H */
