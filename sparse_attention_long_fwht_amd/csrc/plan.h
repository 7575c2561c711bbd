// plan.h -- host-side launch plan and workspace layout shared by the API and the
// kernel launchers.  Internal to libadamas.so (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace adamas {

constexpr int kHeadDim = 128;
constexpr int kCodeBytes = 32;
constexpr int kMaxDist = 384;     // distances 0..384 (128 coordinates x largest code gap 3)
// Selection keys: the distance, or -- when positions are forced -- 0 for a
// forced position and distance + 1 for the others: 0..385.
constexpr int kMaxKey = kMaxDist + 1;
// Sparse path: chunks of the scan (one block per (b, kv head, chunk)).
constexpr int kScanMinChunk = 512;   // = threads of the scan block: one key per thread per pass
constexpr int kScanMaxChunk = 8192;  // at most sixteen passes per block
constexpr int kScanTargetChunks = 64;  // chunks per head wanted at most (see make_plan)
constexpr int64_t kScanBlocks = 256;   // scan blocks wanted at most: one per compute unit
constexpr int64_t kMaxCapacity = 524288;  // positions per (b, kv head)
constexpr int kSelMaxChunks = 128;  // chunks per (b, kv head) at most: kMaxCapacity / 4096
// u16 per (head, chunk) record: the cumulative count of positions at each
// selection key 0..kMaxKey, padded (the padding words repeat the last count)
constexpr int kRecStride = 392;
static_assert(kMaxKey + 1 <= kRecStride, "a record holds every selection key");
static_assert(kRecStride % 8 == 0, "records are copied in 16-byte words");

// Division by a divisor fixed for a launch, without the long integer-division
// sequence: m = div_magic(d) is floor(2^32 / d) (2^32 - 1 for d = 1).  For
// 0 <= n < 2^31, n * m / 2^32 lies in (n / d - 1, n / d], so its integer part
// is floor(n / d) or one less, and one correction step gives floor(n / d).
inline uint32_t div_magic(int d) {
  return d <= 1 ? 0xFFFFFFFFu : (uint32_t)(((uint64_t)1 << 32) / (uint64_t)d);
}
#if defined(__HIP__)
__host__ __device__
#endif
inline int div_by(int n, int d, uint32_t m) {
  uint32_t q = (uint32_t)(((uint64_t)(uint32_t)n * m) >> 32);
  if ((uint32_t)n - q * (uint32_t)d >= (uint32_t)d) ++q;
  return (int)q;
}
// Dense baseline: chunks of the split-K attention.
constexpr int kMaxChunks = 128;      // dense chunks per (b, kv head)
constexpr int kPartFloats = 132;     // m, l, 2 pad, o[128]
// Dynamic LDS the select/attend kernel may take (160 KB per block, less what
// its static arrays need).
constexpr size_t kSelectDynLdsMax = 144 * 1024;
// The single-launch step (scan, hand-off and select/attend in one kernel):
// groups (b, kv head) and chunks per group it serves at most, and its
// synchronisation words at the start of every decode workspace: a generation
// per group, then a 64-bit flag per (group, chunk).
constexpr int kFusedMaxGroups = 64;
constexpr int kFusedMaxChunks = 32;
constexpr size_t kSyncFlagOffset = 256;
constexpr size_t kSyncBytes = kSyncFlagOffset + (size_t)kFusedMaxGroups * kFusedMaxChunks * 8;
static_assert(kFusedMaxGroups * 4 <= (int)kSyncFlagOffset, "the generations fit before the flags");
static_assert(kSyncBytes % 256 == 0, "regions stay 256-byte aligned");

struct Plan {
  int B, Hq, Hkv, R, cap, budget;
  int chunk;           // positions per chunk (power of two)
  int nch;             // chunks covering cap
  int pre_slots;       // leading sorted slots per chunk the select/attend kernel keeps in LDS
  int splits;          // blocks per query head in the select/attend kernel
  int rows_per_split;  // selected rows each of those blocks attends over
  int bitmap_words;    // ceil(cap / 32)
  size_t lds_select;   // dynamic LDS of the select/attend kernel
  bool supported;      // false: the select/attend kernel's LDS would not fit this shape and budget
  bool fused;          // the shape allows the single-launch step (the host also checks residency)
  size_t off_sync, off_sorted, off_rec, off_part, off_count, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int choose_chunk(int cap, int min_chunk, int max_chunks) {
  int c = min_chunk;
  while ((int64_t)c * max_chunks < cap) c <<= 1;
  return c;
}

// Rows per select/attend block (a multiple of the 128-row attention tile).
// Several blocks share a head while the heads alone leave the GPU's compute
// units idle (about kSelectBlocks blocks wanted) or a block would attend more
// than 16 tiles; at most 64 blocks share a head.
constexpr int kSelectBlocks = 256;
inline int choose_rows_per_split(int budget, int heads) {
  int splits = (kSelectBlocks + heads - 1) / heads;
  const int tiles = (budget + 127) / 128;
  splits = splits < 1 ? 1 : (splits > tiles ? tiles : splits);
  splits = splits < (tiles + 15) / 16 ? (tiles + 15) / 16 : splits;
  splits = splits > 64 ? 64 : splits;
  int r = (budget + splits - 1) / splits;
  return (r + 127) / 128 * 128;
}

inline int R_of(int Hq, int Hkv) { return Hkv > 0 ? Hq / Hkv : 1; }

inline Plan make_plan(int B, int Hq, int Hkv, int cap, int budget, bool dense) {
  Plan p{};
  p.supported = true;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.R = Hq / Hkv;
  p.cap = cap;
  p.budget = budget;
  // No step selects more than min(budget, capacity) rows: the launch shape is
  // planned for that (budget itself is only the stride of sel_idx), which also
  // keeps the arithmetic below far from overflow for any int32 budget.
  const int kb = budget < cap ? budget : cap;
  const size_t bhq = (size_t)B * Hq;
  size_t off = 0;
  if (dense) {
    // chunks of at least 1024 positions (each wave of a block then streams 16
    // tiles or more, which amortizes its first loads' latency), doubled while
    // the grid has more than 256 blocks (one per compute unit) or a head more
    // than kMaxChunks chunks.  (Measured: 32K, 256 blocks of 1024 positions
    // 36.8 us against 41.4 for 512 of 512; 128K, 256 blocks 103 us, 512 108,
    // 1024 118; 512K, 256 or 512 blocks 377 us, 1024 385.)
    p.chunk = choose_chunk(cap, 1024, kMaxChunks);
    while ((int64_t)B * Hkv * ((cap + p.chunk - 1) / p.chunk) > 256 && p.chunk < cap) p.chunk <<= 1;
    p.nch = (cap + p.chunk - 1) / p.chunk;
    p.splits = 1;
    p.off_part = off;
    off = align256(off + bhq * p.nch * kPartFloats * sizeof(float));
    p.off_count = off;  // one 64-bit generation word per (b, kv head)
    off = align256(off + (size_t)B * Hkv * sizeof(uint64_t));
    p.total = off;
    return p;
  }
  // chunks grow (up to kScanMaxChunk) until a head has at most
  // kScanTargetChunks of them and the scan grid is about kScanBlocks blocks:
  // larger chunks amortize each block's query encode and record pass
  p.chunk = kScanMinChunk;
  auto scan_blocks = [&](int ch) { return (int64_t)B * Hkv * ((cap + ch - 1) / ch); };
  while (p.chunk < kScanMaxChunk / 2 &&
         ((int64_t)p.chunk * kScanTargetChunks < cap || scan_blocks(p.chunk) > kScanBlocks))
    p.chunk <<= 1;
  // Chunks of 8192 (the sixteen-pass scan) only where they need fewer rounds of
  // resident blocks than chunks of 4096: a round's blocks run their phases in
  // step, so a second, partial round pays every phase's latency again.  Blocks
  // per compute unit: by LDS (160 KB: the R histograms of 448 bins, records,
  // query codes and limits, plus R x chunk sorted slots), at most 4 of 512
  // threads.
  if (p.chunk == kScanMaxChunk / 2) {
    auto rounds = [&](int ch) {
      const int64_t lds = (int64_t)R_of(Hq, Hkv) * (448 * 4 + kRecStride * 2 + 36) + 32 +
                          (int64_t)R_of(Hq, Hkv) * ch * 2;
      int64_t per_cu = 163840 / lds;
      per_cu = per_cu < 1 ? 1 : (per_cu > 4 ? 4 : per_cu);
      const int64_t slots = 256 * per_cu;
      return (scan_blocks(ch) + slots - 1) / slots;
    };
    if (rounds(kScanMaxChunk) < rounds(kScanMaxChunk / 2)) p.chunk = kScanMaxChunk;
  }
  p.nch = (cap + p.chunk - 1) / p.chunk;
  if (p.nch > kSelMaxChunks) p.supported = false;  // (not reached for cap <= kMaxCapacity)
  // about twice the mean number of selected positions per chunk: a power of
  // two, 16..64 (halved below, down to 8, when LDS is short)
  p.pre_slots = 16;
  while (p.pre_slots < 64 && p.pre_slots < 2 * kb / p.nch) p.pre_slots <<= 1;
  p.rows_per_split = choose_rows_per_split(kb, B * Hq);
  p.splits = (kb + p.rows_per_split - 1) / p.rows_per_split;
  p.bitmap_words = ((cap + 31) / 32 + 3) / 4 * 4;  // keeps the record area 16-byte aligned
  // [row list][keep bitmap][sorted prefixes][tie bitmap]; the prefix slots
  // shrink while the LDS is short
  auto lds_for = [&](int pre) {
    return (size_t)p.rows_per_split * sizeof(int) + 2 * (size_t)p.bitmap_words * sizeof(uint32_t) +
           (size_t)p.nch * pre * sizeof(uint16_t);
  };
  while (p.pre_slots > 8 && lds_for(p.pre_slots) > kSelectDynLdsMax) p.pre_slots >>= 1;
  p.lds_select = lds_for(p.pre_slots);
  if (p.lds_select > kSelectDynLdsMax) p.supported = false;
  // single launch: few enough groups and chunks for the sync words, and a
  // block of the group for every (query head, split)
  p.fused = (int64_t)B * Hkv <= kFusedMaxGroups && p.nch <= kFusedMaxChunks && p.R * p.splits <= p.nch &&
            p.chunk <= kScanMaxChunk / 2;  // (the single launch's scan is the eight-pass one)
  p.off_sync = off;
  off += kSyncBytes;
  p.off_sorted = off;
  off = align256(off + bhq * (size_t)p.nch * p.chunk * sizeof(uint16_t));
  p.off_rec = off;
  off = align256(off + bhq * (size_t)p.nch * kRecStride * sizeof(uint16_t));
  p.off_part = off;
  off = align256(off + bhq * p.splits * kPartFloats * sizeof(float));
  p.off_count = off;
  off = align256(off + bhq * sizeof(uint32_t));
  p.total = off;
  return p;
}

// Where the K/V row and the key code of (b, kv head g, position p) live.
// Contiguous caches: row (b * Hkv + g) * cap + p of [B][Hkv][cap].  Paged
// caches: pools [num_pages][Hkv][page][...] and a block table [B][max_pages]
// naming the page of each sequence's positions [j * page, (j + 1) * page);
// the row is (page * Hkv + g) * page_size + p % page_size.  A K or V row starts
// at row * 128 values, a code at row * 32 bytes.
struct KvLayout {
  const int32_t* table;  // paged only
  int max_pages, page_log2, num_pages;
  int Hkv, cap;
  uint32_t hkv_m;  // div_magic(Hkv)
};

#if defined(__HIP__)  // (device code; the plan above also compiles as plain host C++)
template <bool kPaged>
__device__ __forceinline__ size_t kv_row(const KvLayout& L, int b, int g, int p) {
  if (!kPaged) return ((size_t)b * L.Hkv + g) * (size_t)L.cap + (size_t)p;
  // (page ids are a precondition; clamped to the pool all the same)
  const int page = min(max(L.table[(size_t)b * L.max_pages + (p >> L.page_log2)], 0), L.num_pages - 1);
  return ((((size_t)page * L.Hkv + g)) << L.page_log2) + (size_t)(p & ((1 << L.page_log2) - 1));
}
#endif

// Per-thread kernel-timing events (adamas_profile_events).
constexpr int kMaxProfileEvents = 16;
struct ProfileEvents {
  hipEvent_t ev[kMaxProfileEvents];
  int n;
};
ProfileEvents& profile_events();  // this thread's setting
// This thread's decode launch setting (adamas_decode_launch_mode: 1 = single
// launch where possible, 0 = always two kernels) and the number of kernels its
// last decode call launched.
int& launch_mode();
int& launch_count();

// ---- launchers (kernels.hip, decode.hip); kv.table == nullptr: contiguous caches ----
// max_rows > 0: the caller's bound on end[b] - start[b], which sizes the grid
// only (each block walks its range with a stride, so any bound stays correct)
hipError_t launch_encode_keys(int B, const KvLayout& kv, const uint16_t* k, const int32_t* start,
                              const int32_t* end, uint8_t* codes, hipStream_t s, int max_rows = 0);

// Forced positions of a decode step: p < sink, p >= kv_len[b] - recent, or bit
// p % 32 of mask[b * mask_words + p / 32] (mask may be null).  All zero: none.
struct Forced {
  int sink, recent;
  const uint32_t* mask;
  int mask_words;
};

// `append`: first encode the key at position kv_len[b]-1 of every (b, kv head)
// into `codes` (the scan block holding that position does it); otherwise codes
// are only read.
hipError_t launch_decode(const Plan& p, const KvLayout& kv, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, uint8_t* codes, bool append, const Forced& f, const int32_t* kv_len,
                         float scale, float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, char* ws,
                         hipStream_t s);

hipError_t launch_dense(const Plan& p, const KvLayout& kv, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const int32_t* kv_len, float scale, float* out, char* ws,
                        hipStream_t s);

}  // namespace adamas
