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
  int chunk;           // positions per chunk (power of two)
  int nch;             // chunks covering cap
  int dstride;         // distance row stride (positions), multiple of 64
  int splits;          // blocks per query head in the select/attend kernel
  int rows_per_split;  // selected rows each of those blocks attends over
  size_t off_dist, off_hist, off_part, off_count, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Chunk size: the smallest power of two >= kMinChunk that keeps cap within
// kMaxChunks chunks.
inline int choose_chunk(int cap) {
  int c = kMinChunk;
  while ((int64_t)c * kMaxChunks < cap) c <<= 1;
  return c;
}

// Rows per select/attend block: at least 256, and few enough blocks per head
// (<= 64) that merging their partials stays cheap.
inline int choose_rows_per_split(int budget) {
  int r = (budget + 63) / 64;
  r = (r + 127) / 128 * 128;
  return r < 256 ? 256 : r;
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
  p.dstride = (cap + 63) / 64 * 64;
  p.rows_per_split = choose_rows_per_split(budget);
  p.splits = dense ? 1 : (budget + p.rows_per_split - 1) / p.rows_per_split;
  size_t off = 0;
  const size_t bhq = (size_t)B * Hq;
  size_t nparts;
  if (!dense) {
    p.off_dist = off;
    off = align256(off + bhq * (size_t)p.dstride * sizeof(uint16_t));
    p.off_hist = off;
    off = align256(off + bhq * p.nch * kHistStride * sizeof(uint16_t));
    nparts = bhq * p.splits;
  } else {
    nparts = bhq * p.nch;
  }
  p.off_part = off;
  off = align256(off + nparts * kPartFloats * sizeof(float));
  p.off_count = off;
  off = align256(off + bhq * sizeof(uint32_t));
  p.total = off;
  return p;
}

// Per-thread kernel-timing events (adamas_profile_events).
constexpr int kMaxProfileEvents = 16;
struct ProfileEvents {
  hipEvent_t ev[kMaxProfileEvents];
  int n;
};
ProfileEvents& profile_events();  // this thread's setting

// ---- launchers (kernels.hip) ----
hipError_t launch_encode_keys(int B, int Hkv, int cap, const uint16_t* k, const int32_t* start,
                              const int32_t* end, uint8_t* codes, hipStream_t s);

// `append`: first encode the key at position kv_len[b]-1 of every (b, kv head)
// into `codes` (the scan block holding that position does it); otherwise codes
// are only read.
hipError_t launch_decode(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* codes,
                         bool append, const int32_t* kv_len, float scale, float* out, int32_t* sel_idx,
                         uint16_t* dist, uint8_t* q_codes, char* ws, hipStream_t s);

hipError_t launch_dense(const Plan& p, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const int32_t* kv_len, float scale, float* out, char* ws, hipStream_t s);

}  // namespace adamas
