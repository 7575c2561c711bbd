// plan.h -- host-side launch plan and workspace layout shared by the API and the
// kernel launchers.  Internal to libadamas.so (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace adamas {

constexpr int kHeadDim = 128;
constexpr int kCodeBytes = 32;
constexpr int kBins = 385;        // distances 0..384 (128 coordinates x largest code gap 3)
constexpr int kHistStride = 392;  // u16 entries per stored histogram row (784 B, 16 B aligned)
constexpr int kMaxChunks = 128;           // chunks per (batch, kv head)
constexpr int kMinChunk = 512;            // positions per chunk, lower bound
constexpr int kMaxChunk = 8192;           // upper bound (LDS list of one chunk)
constexpr int kPartFloats = 132;          // m, l, 2 pad, o[128]
constexpr int64_t kMaxCapacity = (int64_t)kMaxChunks * kMaxChunk;  // 1,048,576 positions

struct Plan {
  int B, Hq, Hkv, R, cap, budget;
  int chunk;  // positions per chunk (power of two)
  int nch;    // chunks covering cap
  size_t off_dist, off_hist, off_cinfo, off_hinfo, off_part, off_count, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunk size: the smallest power of two >= kMinChunk that keeps cap within
// kMaxChunks chunks.
inline int choose_chunk(int cap) {
  int c = kMinChunk;
  while ((int64_t)c * kMaxChunks < cap) c <<= 1;
  return c;
}

inline Plan make_plan(int B, int Hq, int Hkv, int cap, int budget, bool dense) {
  Plan p{};
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.R = Hq / Hkv;
  p.cap = cap;
  p.budget = budget;
  p.chunk = choose_chunk(cap);
  p.nch = (cap + p.chunk - 1) / p.chunk;
  size_t off = 0;
  const size_t bhq = (size_t)B * Hq;
  if (!dense) {
    p.off_dist = off;
    off = align256(off + bhq * (size_t)cap * sizeof(uint16_t));
    p.off_hist = off;
    off = align256(off + bhq * p.nch * kHistStride * sizeof(uint16_t));
    p.off_cinfo = off;
    off = align256(off + bhq * p.nch * 2 * sizeof(int32_t));
    p.off_hinfo = off;
    off = align256(off + bhq * 2 * sizeof(int32_t));
  }
  p.off_part = off;
  off = align256(off + bhq * p.nch * kPartFloats * sizeof(float));
  p.off_count = off;
  off = align256(off + (size_t)B * Hkv * sizeof(uint32_t));
  p.total = off;
  return p;
}

// ---- launchers (kernels.hip) ----
hipError_t launch_encode_keys(int B, int Hkv, int cap, const uint16_t* k, const int32_t* start,
                              const int32_t* end, uint8_t* codes, hipStream_t s);

hipError_t launch_decode(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint8_t* codes, const int32_t* kv_len, float scale, float* out,
                         int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, char* ws, hipStream_t s);

hipError_t launch_dense(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* kv_len, float scale, float* out, char* ws, hipStream_t s);

}  // namespace adamas
