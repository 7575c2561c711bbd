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
// scan_kernel          one block per (b, kv head, chunk of positions): the
//                      group's R query vectors are encoded (one wave per
//                      vector), then each key code of the chunk is read once and
//                      its distance to all R query codes computed; per (query
//                      head, chunk) a counting sort by distance leaves a record
//                      (cumulative counts per distance up to the chunk's share of
//                      the budget) and the positions ordered by distance.
// select_attend_kernel grid (B*Hq, splits): per query head, the records give the
//                      threshold distance T (the k-th smallest) and how many ties
//                      at T to keep; each chunk's kept positions are emitted in
//                      ascending order into LDS; the block gathers those K/V rows
//                      and runs exact softmax attention (MFMA for q.K, VALU for
//                      P.V).  With several splits each block takes a slice of the
//                      selection and the last one merges the slices' (m, l, o)
//                      partials.
//
// Forced positions (sinks, a recent window, a caller bitmap; the blog's
// sections 3.2 and 6 keep special tokens at full attention) need no change past
// the scan: the scan ranks by a key that is 0 for a forced position and distance
// + 1 for the others, so forced positions come first, in position order, and the
// others follow by (distance, position).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
// 1, 2, 4, ..., 64 as everywhere else.  Every exchange stays in the vector
// ALU (DPP for 1..8, the gfx950 row and half swaps for 16 and 32): no LDS
// round trip on the way to the first distances.  The codes come out as wave
// ballots: bit l of a ballot over coordinate l is exactly the planar packed
// layout.

template <int H>
__device__ __forceinline__ float xor_partner(float v) {
  if constexpr (H == 1) return quad_swap<kQuadXor1>(v);
  else if constexpr (H == 2) return quad_swap<kQuadXor2>(v);
  else if constexpr (H < 32) return __uint_as_float(lane_xor_u32<H>(__float_as_uint(v)));  // (DPP, lane swap: no LDS)
  else return __uint_as_float(xor32_u32(__float_as_uint(v)));  // (gfx950 lane swap, no LDS)
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
// Scan: distances, then a counting sort of each chunk by distance
// --------------------------------------------------------------------------
//
// Per (query head, chunk) the scan leaves two things in the workspace:
//   sorted[slot]  chunk-local positions ordered by distance (any order inside a
//                 distance), kept only for distances <= localk, where localk is
//                 the smallest distance with at least kk = min(k, n_c)
//                 positions at or below it (n_c = positions in the chunk);
//   record        the cumulative count cum(d) of the chunk's positions at
//                 distance <= d, for every d = 0 .. kMaxKey.
// (k = the ranked budget, k_eff less the always-kept positions; "distance"
// means the selection key, which differs from the distance only with forced
// positions.)  Summed over the chunks, the records give the exact count of
// positions at or below every distance, so the threshold T (the k-th smallest
// distance) takes one sum; T never exceeds localk of a chunk with kk = k (that
// chunk alone has k positions at or below localk), and a chunk with kk = n_c
// keeps all of its positions in the sorted slots, so the sorted prefixes hold
// every selected position.

constexpr int kScanThreads = 512;  // one key per thread per pass
// popcount(x) + acc in one instruction.  (Left to itself the compiler sums a
// run of popcounts as a tree of three-input adds, one more instruction per
// three terms; the distance is a run of eight.)
__device__ __forceinline__ uint32_t popc_acc(uint32_t x, uint32_t acc) {
  uint32_t r;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(acc));
  return r;
}

constexpr int kHistBins = 7 * 64;  // bins as scanned by one wave: 7 per lane (up to kMaxKey + 1 used)
// the last bin takes the keys a forced-position scan does not rank (sinks and
// window): counted like the others so that no atomic sits behind a branch, then
// left out of the records and the scatter
constexpr int kSpareBin = kHistBins - 1;
static_assert(kSpareBin > kMaxKey, "every selection key has a bin, and the spare bin is none of them");
constexpr int kScanPasses = kScanMaxChunk / kScanThreads;  // 16
constexpr int kSmallPasses = 8;                             // chunks up to 4096 positions
constexpr int kShortPasses = 2;                             // chunks up to 1024 positions (also 1 and 4)

struct ScanArgs {
  const uint16_t* q;
  const uint16_t* k;   // read only when `append`
  uint8_t* codes;      // read; written only when `append` (the appended key's code)
  const int32_t* kv_len;
  uint16_t* sorted;    // [B][Hq][nch][chunk]
  uint16_t* rec;       // [B][Hq][nch][kRecStride]
  uint16_t* dist_out;  // optional [B][Hq][cap]
  uint8_t* q_codes;    // optional [B][Hq][32]
  uint32_t* counters;  // [B][Hq], cleared here for select_attend_kernel
  const uint32_t* fmask;  // optional [B][fmask_words] bitmap of special tokens (ranked first)
  int Hq, Hkv, cap, chunk, nch, budget, append;
  int sink, recent;    // always-kept sinks and recent window (not ranked)
  int fmask_words;     // (sink, recent, fmask: scan_kernel<R, true> only)
  KvLayout kv;         // where K rows and codes of a position live (scan_kernel<R, F, true>: paged)
  uint32_t nch_m, hkv_m;  // div_magic(nch), div_magic(Hkv)
  int xcd_map;         // the number of groups (b, kv head) is a multiple of kXcds
};

// Blocks are dealt to the eight XCDs round-robin by linear block index.  When
// the number of groups allows it, all chunks of one (b, kv head) group go to the
// same XCD, so the group's query rows are fetched into one L2 only.
constexpr int kXcds = 8;

// The (b, kv head) group and the chunk of scan block `blk` of a grid of
// G * nch blocks (divisions by nch through its magic number: the block's first
// loads wait for this).
__device__ __forceinline__ void scan_block_of(int blk, const ScanArgs& a, int& bg, int& c) {
  if (a.xcd_map) {
    const int xcd = blk & (kXcds - 1), s = (int)((uint32_t)blk / kXcds);
    const int z = div_by(s, a.nch, a.nch_m);
    bg = xcd + kXcds * z;
    c = s - z * a.nch;
  } else {
    bg = div_by(blk, a.nch, a.nch_m);
    c = blk - bg * a.nch;
  }
}

// One scan block: chunk c of group bg.  kForced: sinks / recent window /
// special tokens in use (a separate instantiation, so that the plain step
// pays nothing for them).  kCoherent: the records, sorted prefixes and the
// split counters are written through, for readers in the same kernel (the
// single-launch step); otherwise the kernel boundary hands them over.
template <int R, bool kForced, bool kPaged, bool kCoherent, int kPasses>
__device__ __forceinline__ void scan_chunk(const ScanArgs& a, int bg, int c) {
  const int b = div_by(bg, a.Hkv, a.hkv_m);
  const int g = bg - b * a.Hkv;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int p0 = c * a.chunk;

  // kv_len, then the query rows (wave w < R encodes query w), then the key
  // codes: vector loads complete in order, so a wait for one waits for every
  // one issued before it -- the encode must not wait behind the key codes
  const int len = min(a.kv_len[b], a.cap);  // (kv_len <= capacity is a precondition; clamped all the same)
  const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)(g * R + min(wave, R - 1))) * kHeadDim;
  const uint16_t q_lo = qrow[lane], q_hi = qrow[lane + 64];
  // first pass of key codes, addresses clamped to the capacity so that they
  // do not wait for kv_len
  const uint8_t* cbase = a.codes + (kPaged ? (size_t)0 : (size_t)bg * (size_t)a.cap * kCodeBytes);
  auto code_src = [&](int pp) {
    if constexpr (kPaged) return reinterpret_cast<const uint4*>(a.codes + kv_row<true>(a.kv, b, g, pp) * kCodeBytes);
    else return reinterpret_cast<const uint4*>(cbase + (size_t)pp * kCodeBytes);
  };
  int p = min(p0 + tid, a.cap - 1);
  const uint4* c0 = code_src(p);
  uint4 klo = c0[0];
  uint4 khi = c0[1];

  __shared__ uint32_t s_hist[R][kHistBins];  // counts, then exclusive offsets (bins past kMaxKey stay 0 but for kSpareBin)
  __shared__ uint32_t s_code[R + 1][8];      // query codes, then the appended key's
  __shared__ uint32_t s_limit[R];                    // sorted slots kept per head
  __shared__ __attribute__((aligned(16))) uint16_t s_rec[R][kRecStride];  // records, staged
  extern __shared__ __attribute__((aligned(16))) uint16_t s_sorted[];       // [R][chunk] sorted slots, staged
#pragma unroll
  for (int i0 = 0; i0 < R * kHistBins; i0 += kScanThreads)
    if (i0 + tid < R * kHistBins) (&s_hist[0][0])[i0 + tid] = 0u;
  // Vectors to encode: the group's R queries, plus -- in the block holding
  // position len-1 when appending -- that key.  Wave w takes vectors w, w+8.
  const bool app_here = a.append && (len - 1) >= p0 && (len - 1) < p0 + a.chunk;
  const int nvec = R + (app_here ? 1 : 0);
#pragma unroll 1
  for (int vi = wave; vi < nvec; vi += kScanThreads / 64) {
    uint32_t xlo = q_lo, xhi = q_hi;  // vi < R: vi == wave, the row loaded above
    if (vi >= R) {
      const uint16_t* row = a.k + (kPaged ? kv_row<true>(a.kv, b, g, len - 1)
                                          : (size_t)bg * a.cap + (size_t)(len - 1)) * kHeadDim;
      xlo = row[lane];
      xhi = row[lane + 64];
    }
    uint32_t lo[4], hi[4];
    encode_wave(xlo, xhi, lo, hi);
    // lane j < 8 takes word j of the code: the low plane's four words, then
    // the high plane's (wave-uniform values written into single lanes)
    uint32_t w = lo[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) w = lane == j ? (j < 4 ? lo[j & 3] : hi[j & 3]) : w;
    if (lane < 8) {
      s_code[vi][lane] = w;
      if (vi < R) {
        if (__builtin_expect(c == 0 && a.q_codes != nullptr, 0))
          reinterpret_cast<uint32_t*>(a.q_codes + ((size_t)b * a.Hq + (size_t)(g * R + vi)) * kCodeBytes)[lane] = w;
      } else {
        reinterpret_cast<uint32_t*>(a.codes + (kPaged ? kv_row<true>(a.kv, b, g, len - 1)
                                                      : (size_t)bg * a.cap + (size_t)(len - 1)) * kCodeBytes)[lane] = w;
      }
    }
  }
  if (c == 0 && tid < R) {
    uint32_t* cnt = &a.counters[(size_t)b * a.Hq + g * R + tid];
    if constexpr (kCoherent) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else *cnt = 0u;
  }
  __syncthreads();
  const size_t hc0 = (size_t)(b * a.Hq + g * R) * a.nch + c;  // (head g*R, chunk c)
  if (__builtin_expect(p0 >= len, 0)) {
    // a chunk past the sequence: every count of its records is 0 (the select
    // kernel sums a head's first records without a bound on the chunk)
    if (wave < R && lane < kRecStride / 8)
      st16<kCoherent>(a.rec + (hc0 + (size_t)wave * a.nch) * kRecStride + 8 * lane, make_uint4(0u, 0u, 0u, 0u));
    return;
  }
  const int p1 = min(p0 + a.chunk, len);
  // The sinks [0, s_b) and the recent window [len - r_b, len) are always kept
  // and take no part in the ranking: the chunk ranks its share [m0, m1) (maybe
  // empty) of the middle, for the k_mid = k_eff - s_b - r_b remaining slots.
  const int s_b = kForced ? min(a.sink, len) : 0, r_b = kForced ? min(a.recent, len - s_b) : 0;
  const int m0 = kForced ? max(p0, s_b) : p0, m1 = kForced ? min(p1, len - r_b) : p1;
  const int k_mid = min(a.budget, len) - s_b - r_b;  // >= 0: sink + recent <= budget

  // the query codes' low and high planes (uniform)
  uint32_t ql[R][4], qh[R][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      ql[r][w] = __builtin_amdgcn_readfirstlane(s_code[r][w]);
      qh[r][w] = __builtin_amdgcn_readfirstlane(s_code[r][4 + w]);
    }

  // special tokens (kForced with a mask): the caller's bitmap words of every
  // pass, requested before the first wait on the key codes
  uint32_t fw[kPasses];
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    fw[pass] = 0u;
    if (kForced && a.fmask && p0 + pass * kScanThreads < p1)
      fw[pass] = a.fmask[(size_t)b * a.fmask_words + ((min(p0 + pass * kScanThreads + tid, p1 - 1)) >> 5)];
  }

  // selection keys (the distance; with kForced 0 for a special token,
  // distance + 1 for the other ranked keys and kSpareBin for the unranked);
  // each (key, head) takes the next rank in its key's bin.  The next pass's
  // codes are loaded while this pass computes.
  uint32_t dr[kPasses][R];  // (key << 16) | rank inside the bin
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int base = p0 + pass * kScanThreads;
    if (base < p1) {
      uint4 nlo = klo, nhi = khi;
      if (pass + 1 < kPasses && base + kScanThreads < p1) {
        const int pn = min(base + kScanThreads + tid, p1 - 1);
        const uint4* cn = code_src(pn);
        nlo = cn[0];
        nhi = cn[1];
      }
      p = base + tid;
      // the code this block just produced replaces the stored one (a uniform
      // test first: one block of a group holds position len - 1)
      if (__builtin_expect(app_here && len - 1 - base < kScanThreads && len - 1 >= base, 0)) {
        if (p == len - 1) {
          klo = make_uint4(s_code[R][0], s_code[R][1], s_code[R][2], s_code[R][3]);
          khi = make_uint4(s_code[R][4], s_code[R][5], s_code[R][6], s_code[R][7]);
        }
      }
      if (p < p1) {
        // |a - b| for 2-bit codes a = 2 ha + la, b = 2 hb + lb: its low bit is
        // L = la ^ lb (the parity of a - b) and its high bit M = [|a - b| >= 2]
        // = (ha ^ hb) & ~(L & (ha ^ la)) (the high bits differ and the low
        // difference does not have the opposite sign: checked over all 16
        // pairs), so the sum over the 128 coordinates is
        // popcount(L) + 2 popcount(M), word by word over the bit planes.
        const bool ranked = !kForced || (p >= m0 && p < m1);
        const bool special = kForced && ((fw[pass] >> (p & 31)) & 1u);
        const uint32_t lo[4] = {klo.x, klo.y, klo.z, klo.w};
        const uint32_t hi[4] = {khi.x, khi.y, khi.z, khi.w};
        uint32_t x[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) x[w] = hi[w] ^ lo[w];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t cl = 0, cm = 0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t L = lo[w] ^ ql[r][w];
            const uint32_t M = (hi[w] ^ qh[r][w]) & ~(L & x[w]);
            cl = w == 0 ? (uint32_t)__builtin_popcount(L) : popc_acc(L, cl);
            cm = w == 0 ? (uint32_t)__builtin_popcount(M) : popc_acc(M, cm);
          }
          const uint32_t d = cl + 2u * cm;
          const uint32_t key = kForced ? (!ranked ? (uint32_t)kSpareBin : special ? 0u : d + 1u) : d;
          dr[pass][r] = (key << 16) | atomicAdd(&s_hist[r][key], 1u);
          if (kForced && a.dist_out)
            a.dist_out[((size_t)b * a.Hq + (size_t)(g * R + r)) * (size_t)a.cap + p] = (uint16_t)d;
        }
      }
      klo = nlo;
      khi = nhi;
    }
  }
  __syncthreads();
  // debug distances of the plain step: the key is the distance
  if (__builtin_expect(!kForced && a.dist_out != nullptr, 0)) {
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
      const int pp = p0 + pass * kScanThreads + tid;
      if (p0 + pass * kScanThreads < p1 && pp < p1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          a.dist_out[((size_t)b * a.Hq + (size_t)(g * R + r)) * (size_t)a.cap + pp] = (uint16_t)(dr[pass][r] >> 16);
      }
    }
  }

  // per head (wave r): bin offsets, localk, the slots kept, and the record
  // (cumulative counts; a chunk with nothing to rank has all of them 0).
  const int n_c = max(m1 - m0, 0);
  const int kk = min(k_mid, n_c);
  if (wave < R) {
    // (branch-free: selects instead of a search loop; cross-lane reads in
    // uniform code only -- a value read from lane lk must have been computed
    // with lane lk active)
    const int r = wave;
    uint32_t cnt[7], cum[7], loc = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      cnt[j] = s_hist[r][7 * lane + j];  // bins past kMaxKey are zero, but for the spare bin
      if (kForced && 7 * lane + j == kSpareBin) cnt[j] = 0u;
    }
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      loc += cnt[j];
      cum[j] = loc;  // inclusive, inside the lane
    }
    const uint32_t inc = wave_inclusive_scan_u32(loc);
    const uint32_t base = inc - loc;
    const int lk = __builtin_ffsll((long long)__ballot(inc >= (uint32_t)kk)) - 1;  // total n_c >= kk
    int kj = 7;  // this lane's first bin reaching kk
#pragma unroll
    for (int j = 6; j >= 0; --j) kj = base + cum[j] >= (uint32_t)kk ? j : kj;
    uint32_t lim_l = 0;  // positions up to that bin
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      lim_l = j == kj ? base + cum[j] : lim_l;
      s_hist[r][7 * lane + j] = base + cum[j] - cnt[j];  // exclusive offset of the bin
    }
    // slots kept: every position up to localk, the first key whose cumulative
    // count reaches kk (kk == 0 finds key 0: a prefix nothing selects)
    const uint32_t limit = (uint32_t)__builtin_amdgcn_readlane((int)lim_l, lk);
    if (lane == 0) s_limit[r] = limit;
    // cum(d) for every key d (bins past kMaxKey hold no ranked key: the
    // padding words repeat the chunk's count)
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int d = 7 * lane + j;
      if (d < kRecStride) s_rec[r][d] = (uint16_t)(base + cum[j]);
    }
  }
  __syncthreads();

  // scatter the chunk-local positions, ordered by distance, into LDS: first
  // every slot (bin offset + rank), then every store.  Positions past a
  // head's kept slots are stored too (slots stay below the chunk length);
  // nothing reads them.
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int pp = p0 + pass * kScanThreads + tid;
    if (p0 + pass * kScanThreads < p1 && pp < p1 && (!kForced || (pp >= m0 && pp < m1))) {
#pragma unroll
      for (int r = 0; r < R; ++r) dr[pass][r] = s_hist[r][dr[pass][r] >> 16] + (dr[pass][r] & 0xFFFFu);
    }
  }
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int pp = p0 + pass * kScanThreads + tid;
    if (p0 + pass * kScanThreads < p1 && pp < p1 && (!kForced || (pp >= m0 && pp < m1))) {
#pragma unroll
      for (int r = 0; r < R; ++r) s_sorted[r * a.chunk + dr[pass][r]] = (uint16_t)(pp - p0);
    }
  }
  __syncthreads();

  // copy records and sorted prefixes out in 16-byte words (the words past
  // a head's kept slots carry stale LDS values, which nothing reads)
  if (wave < R && lane < kRecStride / 8) {
    const int r = wave;
    st16<kCoherent>(a.rec + (hc0 + (size_t)r * a.nch) * kRecStride + 8 * lane,
                    reinterpret_cast<const uint4*>(s_rec[r])[lane]);
  }
  const int wlog = __builtin_ctz(a.chunk) - 3;  // log2(16-byte words per chunk)
#pragma unroll 1
  for (int i = tid; i < (R << wlog); i += kScanThreads) {
    const int r = i >> wlog, w = i & ((1 << wlog) - 1);
    if (8 * w < (int)s_limit[r])
      st16<kCoherent>(a.sorted + (hc0 + (size_t)r * a.nch) * a.chunk + 8 * w,
                      reinterpret_cast<const uint4*>(s_sorted + r * a.chunk)[w]);
  }
}

// kPasses: passes of kScanThreads keys per block at most (the chunk divided by
// kScanThreads, rounded up to 8 or 16: the rank array is kPasses x R
// registers and the pass loop is unrolled, so chunks up to 4096 positions get
// the 8-pass kernel)
// The values a block needs before its first loads come first, as scalar
// arguments, which gfx950 preloads into SGPRs when the waves start (the
// library is built with -amdgpu-kernarg-preload-count=16; an aggregate
// argument is not preloaded): the block does not wait for a fetch of its
// arguments before requesting its query rows and key codes.  The rest of the
// arguments stays in the struct.  (32K step: 12.56 -> 12.00 us with both
// kernels so.)
template <int R, bool kForced, bool kPaged, int kPasses>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const uint16_t* q, uint8_t* codes, const int32_t* kv_len,
                                                            int Hq, int Hkv, uint32_t hkv_m, int nch, uint32_t nch_m,
                                                            int xcd_map, int cap, int chunk, ScanArgs a0) {
  ScanArgs a = a0;
  a.q = q;
  a.codes = codes;
  a.kv_len = kv_len;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.hkv_m = hkv_m;
  a.nch = nch;
  a.nch_m = nch_m;
  a.xcd_map = xcd_map;
  a.cap = cap;
  a.chunk = chunk;
  int bg, c;
  scan_block_of((int)blockIdx.x, a, bg, c);
  scan_chunk<R, kForced, kPaged, false, kPasses>(a, bg, c);
}

// --------------------------------------------------------------------------
// Select + gather + attention
// --------------------------------------------------------------------------

struct SelAttArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* kv_len;
  const uint16_t* sorted;  // [B][Hq][nch][chunk]
  const uint16_t* rec;     // [B][Hq][nch][kRecStride]
  float* part;             // [B][Hq][splits][kPartFloats]
  uint32_t* counters;      // [B][Hq]
  int32_t* sel_idx;        // optional [B][Hq][budget]
  float* out;              // [B][Hq][128]
  float qscale;            // softmax scale * log2(e)
  int Hq, Hkv, R, cap, budget, chunk, nch, pre_slots, splits, rows_per_split, bitmap_words;
  int sink, recent;    // always-kept sinks and recent window
  KvLayout kv;         // where K/V rows of a position live (select_attend_kernel<true>: paged)
  uint32_t hq_m;       // div_magic(Hq)
};

constexpr int kSAThreads = 512;
constexpr int kSAWaves = kSAThreads / 64;
constexpr int kSATile = kSAWaves * 16;  // 128 rows per attention tile

// Exclusive prefix sums over the block of two values per thread (every thread
// calls it; each block sum below 2^32), and the block sums.
__device__ __forceinline__ void block_scan2(uint32_t v0, uint32_t v1, uint32_t* s_wsum2, uint32_t& before0,
                                            uint32_t& before1, uint32_t& total0, uint32_t& total1) {
  const int lane = lane_id(), wave = wave_id();
  const uint32_t inc0 = wave_inclusive_scan_u32(v0);
  const uint32_t inc1 = wave_inclusive_scan_u32(v1);
  if (lane == 63) {
    s_wsum2[2 * wave] = inc0;
    s_wsum2[2 * wave + 1] = inc1;
  }
  __syncthreads();
  uint32_t b0 = 0, b1 = 0, t0 = 0, t1 = 0;
#pragma unroll
  for (int w = 0; w < kSAWaves; ++w) {
    const uint32_t x0 = s_wsum2[2 * w], x1 = s_wsum2[2 * w + 1];
    b0 += w < wave ? x0 : 0u;
    b1 += w < wave ? x1 : 0u;
    t0 += x0;
    t1 += x1;
  }
  __syncthreads();
  before0 = b0 + inc0 - v0;
  before1 = b1 + inc1 - v1;
  total0 = t0;
  total1 = t1;
}

// Selection with every chunk's entries in one group of S >= m lanes (see
// select_attend_kernel, step F).
struct SortedEmit {
  uint4 ci[2];             // lane l: chunk 64 g + l of ci[g]: m, lt, first kept rank, ties before it
  const uint16_t* pre;     // LDS sorted prefixes [nch][pre_slots]
  const uint16_t* gsorted; // the head's sorted slots in the workspace
  int pre_slots, chunk, nch_b, len;
  uint32_t quota;
  int lo_rank, hi_rank;
  int c_lo, c_hi;          // the chunks holding ranks of this split (c_lo > c_hi: none)
  int* list;               // LDS rows of this split
  int32_t* sel;            // optional sel_idx row of the head
};

template <int S, bool kCoherent>
__device__ __forceinline__ void emit_sorted(const SortedEmit& e) {
  const int lane = lane_id(), wave = wave_id();
  constexpr int cpi = 64 / S;  // chunks per wave per iteration
  const int j = lane & (S - 1);
  const uint64_t gmask = S == 64 ? ~0ull : (((1ull << S) - 1ull) << (lane & ~(S - 1)));
#pragma unroll 1
  for (int c0 = e.c_lo / cpi * cpi + wave * cpi; c0 <= e.c_hi; c0 += kSAWaves * cpi) {
    const int cc = c0 + lane / S;
    // (c0 .. c0 + cpi - 1 lie in one group of 64 chunks: the group is wave-uniform)
    const uint4 src = c0 < 64 ? e.ci[0] : e.ci[1];
    const int sl = cc & 63;
    uint4 ci;
    ci.x = (uint32_t)__shfl((int)src.x, sl, 64);
    ci.y = (uint32_t)__shfl((int)src.y, sl, 64);
    ci.z = (uint32_t)__shfl((int)src.z, sl, 64);
    ci.w = (uint32_t)__shfl((int)src.w, sl, 64);
    if (cc >= e.nch_b) ci.x = 0u;
    uint32_t key = 0xFFFFFFFFu;
    if (j < (int)ci.x) {
      uint32_t lp = e.pre[(size_t)cc * e.pre_slots + min(j, e.pre_slots - 1)];
      if (j >= e.pre_slots) lp = ld_u16_apart<kCoherent>(e.gsorted + (size_t)cc * e.chunk + j);
      lp = min(lp, (uint32_t)(min(e.chunk, e.len - cc * e.chunk) - 1));  // (a position of the chunk)
      key = ((uint32_t)(cc * e.chunk + (int)lp) << 1) | (j >= (int)ci.y ? 1u : 0u);
    }
    key = group_sort_u32<S>(key);
    const bool valid = key != 0xFFFFFFFFu;
    const bool tie = valid && (key & 1u);
    const uint32_t tie_rank = lanes_below(__ballot(tie) & gmask);
    const bool kept = valid && (!tie || ci.w + tie_rank < e.quota);
    const uint32_t r = ci.z + lanes_below(__ballot(kept) & gmask);
    if (kept && (int)r >= e.lo_rank && (int)r < e.hi_rank) {
      const int pp = (int)(key >> 1);
      e.list[r - e.lo_rank] = pp;
      if (e.sel) e.sel[r] = pp;
    }
  }
}

// Selection, gather and attention of query head bh (b * Hq + h), split
// `split` of its rows.  kCoherent: the records and sorted prefixes were
// written in the same kernel (the single-launch step) and are read coherently.
template <bool kPaged, bool kCoherent>
__device__ __forceinline__ void select_attend_head(const SelAttArgs& a, int bh, int split) {
  const int b = div_by(bh, a.Hq, a.hq_m);
  const int h = bh - b * a.Hq;
  const int g = h >> __builtin_ctz(a.R);  // R is a power of two
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();

  // dynamic LDS: [list: rows_per_split ints][keep bitmap][sorted prefixes: nch x
  // pre_slots u16][tie bitmap]
  extern __shared__ __attribute__((aligned(16))) uint32_t s_dyn[];  // 16-byte aligned: uint4 accesses
  int* s_list = reinterpret_cast<int*>(s_dyn);
  uint32_t* s_keep = s_dyn + a.rows_per_split;
  uint16_t* s_pre = reinterpret_cast<uint16_t*>(s_keep + a.bitmap_words);
  uint32_t* s_tie = s_keep + a.bitmap_words + a.nch * a.pre_slots / 2;

  __shared__ __attribute__((aligned(16))) uint32_t s_hit[kSAWaves][4];  // per wave: ballot of G >= k (2 words), G before its first hit, G at its last lane
  __shared__ uint32_t s_wsum[2 * kSAWaves];
  __shared__ float s_wm[kSAWaves], s_wl[kSAWaves];  // per wave: running max and sum
  __shared__ float s_red[kSAWaves][kHeadDim];
  __shared__ int s_last;

  // ---- A. loads: kv_len, the query fragment, the first pre_slots sorted
  // slots of every chunk and -- thread t for selection key t -- the first
  // records' cumulative counts at key t.  kv_len is a scalar load; an empty
  // asm statement that "redefines" it after those loads keeps every use of it
  // -- and so the wait for it -- behind them.
  int len_raw = a.kv_len[b];
  const int col = lane & 15;
  const int kg = lane >> 4;
  uint4 qf[4];
  {
    const uint16_t* qrow = a.q + (size_t)bh * kHeadDim;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * kg);  // (B operand: q in every column)
  }
  const uint16_t* grec = a.rec + (size_t)bh * a.nch * kRecStride;
  const uint16_t* gsorted = a.sorted + (size_t)bh * a.nch * a.chunk;
  // 16-byte words of sorted prefix per chunk (a power of two)
  const int pper_log2 = __builtin_ctz(a.pre_slots) - 3;
  const int pper = 1 << pper_log2;
  const int p16 = a.nch << pper_log2;
  auto pre_src = [&](int i) {
    const int cc = i >> pper_log2, j = i & (pper - 1);
    return reinterpret_cast<const uint4*>(gsorted + (size_t)cc * a.chunk + 8 * j);
  };
  const uint4 tp = ld16<kCoherent>(pre_src(min(tid, p16 - 1)));  // first pass of the prefixes
  // G(t) = sum over the chunks of cum_c(t): thread t reads key t of every
  // record (one 128-byte line per wave and chunk); the first 32 chunks here.
  // Buffer loads over this head's records: constant offsets (few address
  // instructions), and a chunk past the last reads as zero without a memory
  // access.  The single-launch step reads them coherently instead: a head of
  // 32 chunks or more at constant offsets, a shorter one repeating its last
  // record (both issue the same loads in the same order, so the wait counts
  // after them agree).
  constexpr int kGBatch = 32;
  const uint16_t* gcol = grec + min(tid, kMaxKey);
  const uint32_t gcol_b = 2u * (uint32_t)min(tid, kMaxKey);
  uint32_t cv[kGBatch];
  if constexpr (!kCoherent) {
    const auto rrec = buffer_over(grec, (uint32_t)a.nch * (kRecStride * 2));
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) cv[u] = __builtin_amdgcn_raw_buffer_load_b16(rrec, gcol_b + u * (kRecStride * 2), 0, 0);
  } else if (a.nch >= kGBatch) {
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) cv[u] = ld_u16<kCoherent>(gcol + u * kRecStride);
  } else {
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) cv[u] = ld_u16<kCoherent>(gcol + (size_t)min(u, a.nch - 1) * kRecStride);
  }
  // (in the single-launch step kv_len is loaded long before, by the scan)
  if constexpr (!kCoherent) asm volatile("" : "+s"(len_raw));
  const int len = min(len_raw, a.cap);  // (kv_len <= capacity is a precondition; clamped all the same)
  if (__builtin_expect(len <= 0, 0)) {  // no cached position: nothing selected, attention over the empty set is the zero vector
    if (split == 0 && tid < kHeadDim) a.out[(size_t)bh * kHeadDim + tid] = 0.f;
    if (a.sel_idx)
      for (int64_t i = (int64_t)split * kSAThreads + tid; i < a.budget; i += (int64_t)a.splits * kSAThreads)
        a.sel_idx[(size_t)bh * a.budget + i] = -1;
    return;
  }
  const int k_eff = min(a.budget, len);
  // Final ranks (ascending positions): the sinks [0, s_b), then the k_mid
  // ranked positions, then the recent window; the ranking below works on
  // ranks of the middle (the scan left sinks and window out of it).
  const int s_b = min(a.sink, len), r_b = min(a.recent, len - s_b);
  const int k_mid = k_eff - s_b - r_b;
  const int lo_rank = split * a.rows_per_split;
  const int hi_rank = min(lo_rank + a.rows_per_split, k_eff);
  const int mlo = lo_rank - s_b, mhi = hi_rank - s_b;  // this split's window of middle ranks
  // K and V rows of a position of this head's kv head: Kg + kvoff(p), Vg + kvoff(p)
  const size_t kv_base = kPaged ? (size_t)0 : ((size_t)b * a.Hkv + g) * (size_t)a.cap * kHeadDim;
  const uint16_t* Kg = a.k + kv_base;
  const uint16_t* Vg = a.v + kv_base;
  auto kvoff = [&](int pp) -> size_t {
    if constexpr (kPaged) return kv_row<true>(a.kv, b, g, pp) * kHeadDim;
    else return (size_t)pp * kHeadDim;
  };
  // the split's always-kept row of this thread (-1: none): known from kv_len alone
  int forced_pos = -1;
  if (__builtin_expect(a.sink > 0 || a.recent > 0, 0)) {
    const int i = lo_rank + tid, j = i - s_b;
    if (i < hi_rank && (j < 0 || j >= k_mid)) forced_pos = j < 0 ? i : len - r_b + (j - k_mid);
  }
  const int nch_b = (len + a.chunk - 1) >> __builtin_ctz(a.chunk);  // chunk is a power of two
  reinterpret_cast<uint4*>(s_pre)[min(tid, p16 - 1)] = tp;
#pragma unroll 1
  for (int i = tid + kSAThreads; i < p16; i += kSAThreads) reinterpret_cast<uint4*>(s_pre)[i] = ld16<kCoherent>(pre_src(i));

  // ---- B. threshold.  G(t) is the exact number of ranked positions at key
  // <= t, non-decreasing, and G(kMaxKey) >= k_mid; the threshold T is the
  // smallest key with G(T) >= k_mid, and quota = k_mid - G(T - 1) of the
  // positions at key T are kept (the lowest ones).  Each wave ballots its 64
  // keys; the first wave with a hit holds T.
  // (the scan writes all-zero records for the chunks past the sequence, and
  // the buffer loads read zeros past the last chunk, so only the coherent
  // reads of fewer than 32 chunks need a mask)
  uint32_t G = 0;
  if (!kCoherent || a.nch >= kGBatch) {
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) G += cv[u];
  } else {
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) G += u < nch_b ? cv[u] : 0u;
  }
#pragma unroll 1
  for (int c0 = kGBatch; __builtin_expect(c0 < nch_b, 0); c0 += kGBatch) {  // (more than 32 chunks)
    if constexpr (!kCoherent) {
      const auto rrec = buffer_over(grec, (uint32_t)a.nch * (kRecStride * 2));
#pragma unroll
      for (int u = 0; u < kGBatch; ++u)
        G += __builtin_amdgcn_raw_buffer_load_b16(rrec, gcol_b + (c0 + u) * (kRecStride * 2), 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < kGBatch; ++u) cv[u] = ld_u16<kCoherent>(gcol + (size_t)min(c0 + u, nch_b - 1) * kRecStride);
#pragma unroll
      for (int u = 0; u < kGBatch; ++u) G += c0 + u < nch_b ? cv[u] : 0u;
    }
  }
  {
    const uint64_t hit = __ballot(tid <= kMaxKey && G >= (uint32_t)k_mid);
    const int first = hit ? __builtin_ctzll(hit) : 0;
    const uint32_t g_prev = (uint32_t)__builtin_amdgcn_readlane((int)G, max(first - 1, 0));
    const uint32_t g_last = (uint32_t)__builtin_amdgcn_readlane((int)G, 63);
    if (lane == 0) {
      s_hit[wave][0] = (uint32_t)hit;
      s_hit[wave][1] = (uint32_t)(hit >> 32);
      s_hit[wave][2] = first > 0 ? g_prev : 0u;
      s_hit[wave][3] = g_last;
    }
  }
  __syncthreads();
  // lane w < 8 of every wave reads wave w's entry (one LDS round trip); the
  // first wave with a hit holds T
  int T = kMaxKey;
  uint32_t g_before = (uint32_t)k_mid;  // (kept if no key reaches k_mid: contradictory records)
  {
    const uint4 hw = reinterpret_cast<const uint4*>(&s_hit[0][0])[lane & (kSAWaves - 1)];
    const uint64_t any = __ballot(lane < kSAWaves && (hw.x | hw.y) != 0u);
    const uint32_t hx = (uint32_t)__builtin_amdgcn_readlane((int)hw.x, any ? __builtin_ctzll(any) : 0);
    const uint32_t hy = (uint32_t)__builtin_amdgcn_readlane((int)hw.y, any ? __builtin_ctzll(any) : 0);
    const uint32_t hz = (uint32_t)__builtin_amdgcn_readlane((int)hw.z, any ? __builtin_ctzll(any) : 0);
    const int wp = any ? max(__builtin_ctzll(any) - 1, 0) : 0;
    const uint32_t prev_last = (uint32_t)__builtin_amdgcn_readlane((int)hw.w, wp);
    if (any) {  // (wave-uniform)
      const int w = __builtin_ctzll(any);
      const int first = __builtin_ctzll((uint64_t)hx | ((uint64_t)hy << 32));
      T = 64 * w + first;
      g_before = first > 0 ? hz : (w > 0 ? prev_last : 0u);
    }
  }
  const uint32_t quota = (uint32_t)k_mid - min(g_before, (uint32_t)k_mid);
  // cum(T) and cum(T - 1) of the chunks of lane l (l and 64 + l), for E
  const bool two_groups = nch_b > 64;  // (wave-uniform) chunks 64.. exist
  uint32_t mv[2] = {0u, 0u}, lv[2] = {0u, 0u};
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    if (gi == 1 && __builtin_expect(!two_groups, 1)) break;
    if constexpr (!kCoherent) {  // (a lane past the last chunk reads zeros)
      const auto rrec = buffer_over(grec, (uint32_t)a.nch * (kRecStride * 2));
      const uint32_t ro = (uint32_t)(64 * gi + lane) * (kRecStride * 2);
      mv[gi] = __builtin_amdgcn_raw_buffer_load_b16(rrec, ro, 2 * T, 0);
      lv[gi] = __builtin_amdgcn_raw_buffer_load_b16(rrec, ro, 2 * max(T - 1, 0), 0);
    } else {
      const size_t ro = (size_t)min(64 * gi + lane, nch_b - 1) * kRecStride;
      mv[gi] = ld_u16<kCoherent>(grec + ro + T);
      lv[gi] = ld_u16<kCoherent>(grec + ro + max(T - 1, 0));
    }
  }

  // ---- E. per chunk (every wave, lane l: chunks l and 64 + l): lt =
  // positions below T (slots [0, lt) of its sorted prefix) and m = lt + its
  // positions at T (the next slots).  Ties are kept in position order, so a
  // chunk's first kept rank is (positions below T in earlier chunks) +
  // min(ties in earlier chunks, quota).
  uint4 ci[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
  uint32_t max_m;
  {
    uint32_t lt_carry = 0, tie_carry = 0, mm = 0;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      if (gi == 1 && __builtin_expect(!two_groups, 1)) break;
      const int cc = 64 * gi + lane;
      // (clamps keep any workspace content in bounds: m <= the chunk's positions)
      const uint32_t n = cc < nch_b ? (uint32_t)min(a.chunk, len - cc * a.chunk) : 0u;
      const uint32_t m = min(mv[gi], n);
      const uint32_t lt = T > 0 ? min(lv[gi], m) : 0u;
      const uint32_t lt_inc = wave_inclusive_scan_u32(lt), tie_inc = wave_inclusive_scan_u32(m - lt);
      const uint32_t ltb = lt_carry + lt_inc - lt, tb = tie_carry + tie_inc - (m - lt);
      ci[gi] = make_uint4(m, lt, ltb + min(tb, quota), tb);
      lt_carry += (uint32_t)__builtin_amdgcn_readlane((int)lt_inc, 63);
      tie_carry += (uint32_t)__builtin_amdgcn_readlane((int)tie_inc, 63);
      mm = max(mm, m);
    }
    max_m = (uint32_t)wave_max((float)mm);  // exact: m <= 4096
  }

  // ---- prefetch of the always-kept row of this thread.  (Issued only now:
  // a conditional load earlier would make every later wait on a record or
  // prefix load wait for these rows as well -- vector loads return in order
  // and the wait counts of both paths are merged.)
  uint32_t pe[4] = {0u, 0u, 0u, 0u};
  if (forced_pos >= 0) {
    const size_t row = kvoff(forced_pos);
    pe[0] = *reinterpret_cast<const uint32_t*>(Kg + row);
    pe[1] = *reinterpret_cast<const uint32_t*>(Kg + row + 64);
    pe[2] = *reinterpret_cast<const uint32_t*>(Vg + row);
    pe[3] = *reinterpret_cast<const uint32_t*>(Vg + row + 64);
  }

  // ---- prefetch.  Every kept row lies in slots [0, m) of its chunk's sorted
  // prefix.  For the chunks that hold ranks of this split, one word of each
  // 128-byte line of those K and V rows is loaded now, so that the gather
  // after the ordered emission below finds the rows in L2.  Nothing reads the
  // words until the block's last instructions (pf_sink), so nothing waits for
  // these loads before the gather does.  Wave w takes slots w and w + 8 (within
  // the LDS prefix); lane l chunks l and 64 + l.
  uint32_t pf[2][2][4] = {};
  int c_lo = 1 << 30, c_hi = -1;  // the chunks holding ranks of this split (kept ranks grow with the chunk)
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    if (gi == 1 && __builtin_expect(!two_groups, 1)) break;
    const int cc = 64 * gi + lane;
    const uint4 c = ci[gi];
    const uint32_t kept = c.y + min(c.x - c.y, quota > c.w ? quota - c.w : 0u);  // lt + kept ties
    const bool mine = cc < nch_b && kept > 0u && (int)c.z < mhi && (int)(c.z + kept) > mlo;
    const uint64_t mb = __ballot(mine);
    if (mb) {
      c_lo = min(c_lo, 64 * gi + __builtin_ctzll(mb));
      c_hi = max(c_hi, 64 * gi + 63 - __builtin_clzll(mb));
    }
    // slots [0, lt) are all kept; the ties at T, slots [lt, m), are kept in
    // position order across the chunks, so a chunk keeps all, some (one chunk
    // per head) or none of them -- with none kept they are not prefetched
    const int pf_n = kept > c.y ? (int)c.x : (int)c.y;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = wave + kSAWaves * jj;
      if (mine && j < pf_n && j < a.pre_slots) {
        const int lp = min((int)s_pre[(size_t)cc * a.pre_slots + j], min(a.chunk, len - cc * a.chunk) - 1);
        const size_t row = kvoff(cc * a.chunk + lp);
        pf[gi][jj][0] = *reinterpret_cast<const uint32_t*>(Kg + row);
        pf[gi][jj][1] = *reinterpret_cast<const uint32_t*>(Kg + row + 64);
        pf[gi][jj][2] = *reinterpret_cast<const uint32_t*>(Vg + row);
        pf[gi][jj][3] = *reinterpret_cast<const uint32_t*>(Vg + row + 64);
      }
    }
  }

  if (__builtin_expect(max_m <= 64, 1)) {
    // ---- F. every chunk's m entries in one group of S >= m lanes, sorted by
    // position (key = 2 * position + [at T]); a tie is kept while its rank
    // among all ties stays below the quota; ranks by ballot.  Groups of 8 at
    // least: with at most 128 chunks that is two rounds of the block's waves,
    // and each group width is one more copy of the emission in the kernel's
    // code, which the compute unit fetches cold on every launch (dropping the
    // widths 1, 2 and 4 cut the 32K step by 0.12 us).
    const SortedEmit e{{ci[0], ci[1]}, s_pre, gsorted, a.pre_slots, a.chunk, nch_b, len, quota, mlo, mhi,
                       c_lo, c_hi, s_list, a.sel_idx ? a.sel_idx + (size_t)bh * a.budget + s_b : nullptr};
    if (max_m <= 8) emit_sorted<8, kCoherent>(e);
    else if (max_m <= 16) emit_sorted<16, kCoherent>(e);
    else if (max_m <= 32) emit_sorted<32, kCoherent>(e);
    else emit_sorted<64, kCoherent>(e);
  } else {
    // ---- F (wide chunks). Mark the selected positions in bitmaps with one
    // bit per position: below T -> keep, at T -> tie.  Wave w takes the chunks
    // cc = w (mod 8); a chunk's m entries go one per lane.
    for (int i = tid; i < a.bitmap_words; i += kSAThreads) {
      s_keep[i] = 0u;
      s_tie[i] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      uint64_t rest = __ballot((lane & (kSAWaves - 1)) == wave && 64 * gi + lane < nch_b && ci[gi].x > 0u);
      while (rest) {
        const int i = __builtin_ctzll(rest);
        rest &= rest - 1;
        const int cc = 64 * gi + i;
        const int m = __builtin_amdgcn_readlane((int)ci[gi].x, i), lt = __builtin_amdgcn_readlane((int)ci[gi].y, i);
#pragma unroll 1
        for (int jj = lane; jj < m; jj += 64) {
          uint32_t lp = s_pre[(size_t)cc * a.pre_slots + min(jj, a.pre_slots - 1)];
          if (jj >= a.pre_slots) lp = ld_u16_apart<kCoherent>(gsorted + (size_t)cc * a.chunk + jj);
          const int pp = cc * a.chunk + min((int)lp, min(a.chunk, len - cc * a.chunk) - 1);
          atomicOr((jj < lt ? s_keep : s_tie) + (pp >> 5), 1u << (pp & 31));
        }
      }
    }
    __syncthreads();

    // ---- G/H. keep every position below T and the `quota` lowest positions
    // at T, and emit the kept positions in ascending order: each thread owns
    // contiguous bitmap words; one scan of (kept-below, ties) counts gives each
    // thread its first rank and its share of the quota.
    const int wpt = (a.bitmap_words + kSAThreads - 1) / kSAThreads;  // words per thread
    const int w0 = tid * wpt;
    const int w1 = min(w0 + wpt, a.bitmap_words);
    uint32_t nk = 0, nt = 0;
    for (int w = w0; w < w1; ++w) {
      nk += __builtin_popcount(s_keep[w]);
      nt += __builtin_popcount(s_tie[w]);
    }
    uint32_t kb, tb, ktot, ttot;
    block_scan2(nk, nt, s_wsum, kb, tb, ktot, ttot);
    uint32_t tie_left = tb >= quota ? 0u : min(nt, quota - tb);  // this thread's kept ties
    uint32_t r = kb + min(tb, quota);
    if ((int)r < mhi && (int)(r + nk + tie_left) > mlo) {
      for (int w = w0; w < w1; ++w) {
        uint32_t tw = s_tie[w];
        uint32_t ties_kept = 0;
        while (tw && tie_left) {  // the lowest tie_left ties of this word
          const uint32_t bit = tw & (0u - tw);
          tw ^= bit;
          ties_kept |= bit;
          --tie_left;
        }
        uint32_t bits = s_keep[w] | ties_kept;
        while (bits) {
          const int bit = __builtin_ctz(bits);
          bits &= bits - 1;
          if ((int)r >= mlo && (int)r < mhi) {
            const int pp = 32 * w + bit;
            s_list[r - mlo] = pp;
            if (a.sel_idx) a.sel_idx[(size_t)bh * a.budget + s_b + r] = pp;
          }
          ++r;
        }
      }
    }
  }
  // the always-kept rows of this split: sinks first, the window last
  if (forced_pos >= 0) {
    s_list[tid] = forced_pos;
    if (a.sel_idx) a.sel_idx[(size_t)bh * a.budget + lo_rank + tid] = forced_pos;
  }
  for (int i = lo_rank + kSAThreads + tid; i < hi_rank; i += kSAThreads) {  // (splits over 512 rows)
    const int j = i - s_b;
    if (j >= 0 && j < k_mid) continue;
    const int pp = j < 0 ? i : len - r_b + (j - k_mid);
    s_list[i - lo_rank] = pp;
    if (a.sel_idx) a.sel_idx[(size_t)bh * a.budget + i] = pp;
  }
  if (a.sel_idx) {
    // -1 past k_eff, spread over the head's splits (64-bit indices: budget may
    // be any positive int32)
    for (int64_t i = (int64_t)k_eff + (int64_t)split * kSAThreads + tid; i < a.budget;
         i += (int64_t)a.splits * kSAThreads)
      a.sel_idx[(size_t)bh * a.budget + i] = -1;
  }
  const int nrows = max(0, hi_rank - lo_rank);
  __syncthreads();

  // ---- I. attention over the split's rows: tiles of 128 rows, 16 per wave.
  // Each wave keeps its own running max, sum and output over its rows.
  // Scores: the rows (A operand, lane (col, kg) holds row col's k-range 8 kg
  // of each 32) times q in every column (B operand) give C[r][j] = score of
  // row r for every j, so lane (col, kg) holds the scores of rows 4 kg + i in
  // acc[i] -- the rows whose V it multiplies (dims 8 col .. 8 col + 7).
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = 0.f;
  float m_w = -INFINITY, l_w = 0.f;
  // K and V of the wave's rows of tile t0 (rows past nrows read a valid row;
  // their scores are masked)
  // (a contiguous cache: buffer loads over the kv head's rows, 32-bit offsets)
  [[maybe_unused]] const auto kbuf = buffer_over(Kg, (uint32_t)a.cap * (kHeadDim * 2));
  [[maybe_unused]] const auto vbuf = buffer_over(Vg, (uint32_t)a.cap * (kHeadDim * 2));
  auto gather = [&](int t0, uint4 (&ka)[4], uint4 (&vv)[4]) {
    const int r0 = t0 + 16 * wave;
    const int ia = r0 + col;
    const int pa = min(max(s_list[ia < nrows ? ia : 0], 0), len - 1);  // (clamped: a position of the cache)
    if constexpr (kPaged) {
      const uint16_t* kr = Kg + kvoff(pa) + 8 * kg;
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = *reinterpret_cast<const uint4*>(kr + 32 * s);
    } else {
      const uint32_t ko = (uint32_t)pa * (kHeadDim * 2) + 16 * kg;
#pragma unroll
      for (int s = 0; s < 4; ++s) ka[s] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(kbuf, ko + 64 * s, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int iv = r0 + 4 * kg + i;
      const int pv = min(max(s_list[iv < nrows ? iv : 0], 0), len - 1);
      if constexpr (kPaged)
        vv[i] = *reinterpret_cast<const uint4*>(Vg + kvoff(pv) + 8 * col);
      else
        vv[i] = as_uint4(__builtin_amdgcn_raw_buffer_load_b128(vbuf, (uint32_t)pv * (kHeadDim * 2) + 16 * col, 0, 0));
    }
  };
  uint4 ka[4], vv[4];
  if (nrows > 0) gather(0, ka, vv);
#pragma unroll 1
  for (int t0 = 0; t0 < nrows; t0 += kSATile) {
    const int r0 = t0 + 16 * wave;  // the wave's first row
    uint4 kn[4], vn[4];  // the next tile's rows, requested before this tile is used
    if (t0 + kSATile < nrows) gather(t0 + kSATile, kn, vn);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_16x16x32_bf16(ka[s], qf[s], acc);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = r0 + 4 * kg + i < nrows ? acc[i] * a.qscale : -INFINITY;
    // tile max and sum over the 16 rows: the four of this lane, then across
    // the wave's four 16-lane rows (lane swaps)
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, __uint_as_float(xor16_u32(__float_as_uint(mx))));
    mx = fmaxf(mx, __uint_as_float(xor32_u32(__float_as_uint(mx))));
    const float m_new = fmaxf(m_w, mx);
    if (m_new != -INFINITY) {  // (wave-uniform) the wave has rows
      const float corr = __builtin_amdgcn_exp2f(m_w - m_new);  // 0 while m_w is -inf
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = sc[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - m_new);
      float ls = (pr[0] + pr[1]) + (pr[2] + pr[3]);
      ls += __uint_as_float(xor16_u32(__float_as_uint(ls)));
      ls += __uint_as_float(xor32_u32(__float_as_uint(ls)));
      l_w = __builtin_fmaf(l_w, corr, ls);
      m_w = m_new;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] *= corr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t vw[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          o[2 * j] = __builtin_fmaf(pr[i], bf16_lo(vw[j]), o[2 * j]);
          o[2 * j + 1] = __builtin_fmaf(pr[i], bf16_hi(vw[j]), o[2 * j + 1]);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      ka[s] = kn[s];
      vv[s] = vn[s];
    }
  }
  // ---- J. merge: o over the four k-groups of each wave (its four rows of
  // 16 lanes), then the waves' (max, sum, output) partials.  Two values go
  // through each row swap: swapping o[2p] with o[2p + 1] across rows 0/1 and
  // 2/3 and adding leaves o[2p] summed over a row pair in rows 0 and 2 and
  // o[2p + 1] in rows 1 and 3; the same across the wave halves then leaves
  // the sum of o[kg] over all four rows, (row 0 + row 1) + (row 2 + row 3),
  // in lane (col, kg) of t[0], and of o[4 + kg] in t[1].
  float t[2];
  {
    float s4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(o[2 * q]), __float_as_uint(o[2 * q + 1]),
                                                      false, false);
      s4[q] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(s4[2 * q]), __float_as_uint(s4[2 * q + 1]),
                                                      false, false);
      t[q] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  }
  s_red[wave][8 * col + kg] = t[0];
  s_red[wave][8 * col + 4 + kg] = t[1];
  if (lane == 0) {
    s_wm[wave] = m_w;
    s_wl[wave] = l_w;
  }
  __syncthreads();
  float* pc = a.part + ((size_t)bh * a.splits + split) * kPartFloats;
  if (tid < kHeadDim) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kSAWaves; ++w) M = fmaxf(M, s_wm[w]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kSAWaves; ++w) {
      const float mw = s_wm[w];
      const float wgt = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L = __builtin_fmaf(s_wl[w], wgt, L);
      O = __builtin_fmaf(s_red[w][tid], wgt, O);
    }
    if (a.splits == 1) {
      a.out[(size_t)bh * kHeadDim + tid] = O * __builtin_amdgcn_rcpf(L);
    } else {
      // several splits: publish (m, l, o) write-through; the last split of
      // this head merges them
      store_coherent(pc + 4 + tid, O);
      if (tid == 0) {
        store_coherent(pc, M);
        store_coherent(pc + 1, L);
      }
    }
  }
  {
    // (the prefetched words are used only here, by a test that cannot pass:
    // the budget is positive)
    uint32_t pf_sink = 0;
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int u = 0; u < 4; ++u) pf_sink ^= pf[gi][jj][u];
#pragma unroll
    for (int u = 0; u < 4; ++u) pf_sink ^= pe[u];
    if (a.budget < 0) a.out[tid] = (float)pf_sink;
  }
  if (a.splits == 1) return;
  wait_memory();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&a.counters[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(a.splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (tid < kHeadDim) {
    // (m, l and o of the first eight splits are requested in one round; with
    // more splits, the max over the rest takes one more round first)
    const float* p0 = a.part + (size_t)bh * a.splits * kPartFloats;
    float mv[8], lv[8], ov[8];
    auto load_batch = [&](int s0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* ps = p0 + (size_t)min(s0 + u, a.splits - 1) * kPartFloats;
        mv[u] = load_coherent(ps);
        lv[u] = load_coherent(ps + 1);
        ov[u] = load_coherent(ps + 4 + tid);
      }
    };
    load_batch(0);
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, mv[u]);
#pragma unroll 1
    for (int s0 = 8; s0 < a.splits; s0 += 8) {
      float mm[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) mm[u] = load_coherent(p0 + (size_t)min(s0 + u, a.splits - 1) * kPartFloats);
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, mm[u]);
    }
    float L = 0.f, O = 0.f;
#pragma unroll 1
    for (int s0 = 0; s0 < a.splits; s0 += 8) {
      if (s0 > 0) load_batch(s0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (s0 + u < a.splits && mv[u] != -INFINITY) {
          const float wgt = __builtin_amdgcn_exp2f(mv[u] - M);
          L = __builtin_fmaf(lv[u], wgt, L);
          O = __builtin_fmaf(ov[u], wgt, O);
        }
      }
    }
    a.out[(size_t)bh * kHeadDim + tid] = O * __builtin_amdgcn_rcpf(L);
  }
}

// (at most 128 VGPRs: two blocks of 512 threads per compute unit, which the
// batched shapes need to run their blocks in one round)
template <bool kPaged>
__global__ __launch_bounds__(kSAThreads) __attribute__((amdgpu_waves_per_eu(4))) void select_attend_kernel(
    const uint16_t* q, const uint16_t* rec, const uint16_t* sorted, const int32_t* kv_len, int Hq, uint32_t hq_m,
    int nch, int pre_slots, int chunk, SelAttArgs a0) {
  // (the leading arguments are preloaded into SGPRs, as for scan_kernel)
  SelAttArgs a = a0;
  a.q = q;
  a.rec = rec;
  a.sorted = sorted;
  a.kv_len = kv_len;
  a.Hq = Hq;
  a.hq_m = hq_m;
  a.nch = nch;
  a.pre_slots = pre_slots;
  a.chunk = chunk;
  select_attend_head<kPaged, false>(a, (int)blockIdx.x, (int)blockIdx.y);
}

// --------------------------------------------------------------------------
// Single launch: scan, hand-off, select + attend
// --------------------------------------------------------------------------
//
// Every block scans its chunk (scan_chunk, records and sorted prefixes written
// through), then publishes a flag for that chunk: a 64-bit hash of (generation
// + 1, group, chunk).  The group's first R * splits blocks then take one
// (query head, split) each: they wait until every chunk of the group has
// published (polling the flags with coherent loads, bounded) and run
// select_attend_head, which reads the records coherently.  This replaces the
// kernel boundary between the two kernels (its drain and the second kernel's
// start-up), and needs no assumption about which XCD a block runs on.
//
// The generation of a group is read by every block of the group at its start
// and advanced by the group's first block once it has seen all the flags, so
// each call expects new flag values: flags of an earlier call, or any other
// content of the workspace, do not match (a 64-bit hash).  Every block of the
// grid must be resident at once (the host checks the occupancy), so a waiting
// block never holds a compute unit that a block it waits for needs.

struct FusedSync {
  uint32_t* gen;                // [kFusedMaxGroups]
  unsigned long long* flags;    // [kFusedMaxGroups][kFusedMaxChunks]
};

__device__ __forceinline__ unsigned long long flag_value(uint32_t gen, int bg, int c) {
  // (a splitmix64 finalizer)
  unsigned long long z = ((unsigned long long)gen << 32) ^ ((unsigned long long)bg << 8) ^ (unsigned long long)c;
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

constexpr int kFusedPollMax = 1 << 21;  // about a second of polling: then the head is given up (NaN output)

template <int R, bool kForced, bool kPaged>
// (the scan's first values as preloaded leading arguments, as for scan_kernel)
__global__ __launch_bounds__(kScanThreads) void fused_decode_kernel(const uint16_t* q, uint8_t* codes,
                                                                    const int32_t* kv_len, int Hq, int Hkv,
                                                                    uint32_t hkv_m, int nch, uint32_t nch_m,
                                                                    int xcd_map, int cap, int chunk, ScanArgs sa0,
                                                                    SelAttArgs aa, FusedSync fs) {
  ScanArgs sa = sa0;
  sa.q = q;
  sa.codes = codes;
  sa.kv_len = kv_len;
  sa.Hq = Hq;
  sa.Hkv = Hkv;
  sa.hkv_m = hkv_m;
  sa.nch = nch;
  sa.nch_m = nch_m;
  sa.xcd_map = xcd_map;
  sa.cap = cap;
  sa.chunk = chunk;
  int bg, c;
  scan_block_of((int)blockIdx.x, sa, bg, c);
  __shared__ uint32_t s_gen;
  __shared__ int s_ok;
  if (threadIdx.x == 0) s_gen = __hip_atomic_load(&fs.gen[bg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  scan_chunk<R, kForced, kPaged, true, kSmallPasses>(sa, bg, c);  // (the single launch takes chunks up to 4096)
  wait_memory();    // this thread's written-through stores have completed
  __syncthreads();  // ... and every thread's (s_gen is visible too)
  const uint32_t gen = s_gen;
  if (threadIdx.x == 0)
    __hip_atomic_store(&fs.flags[bg * kFusedMaxChunks + c], flag_value(gen + 1, bg, c), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  // chunk c of the group serves query head c / splits of the group, split c % splits
  const int role = c;
  if (role >= R * aa.splits) return;
  if (threadIdx.x < 64) {
    const int lane = (int)threadIdx.x;
    const bool mine = lane < sa.nch;
    const unsigned long long want = mine ? flag_value(gen + 1, bg, lane) : 0ull;
    bool done = false;
#pragma unroll 1
    for (int it = 0; it < kFusedPollMax; ++it) {
      const unsigned long long f =
          mine ? __hip_atomic_load(&fs.flags[bg * kFusedMaxChunks + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : want;
      if (__ballot(f != want) == 0ull) {
        done = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (lane == 0) s_ok = done ? 1 : 0;
  }
  __syncthreads();
  if (role == 0 && threadIdx.x == 0)
    __hip_atomic_store(&fs.gen[bg], gen + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int b = div_by(bg, sa.Hkv, sa.hkv_m), g = bg - b * sa.Hkv;
  // (readfirstlane: block-uniform values, kept in scalar registers)
  const int bh = __builtin_amdgcn_readfirstlane(b * sa.Hq + g * R + role / aa.splits);
  const int split = __builtin_amdgcn_readfirstlane(role % aa.splits);
  if (!__builtin_amdgcn_readfirstlane(s_ok)) {  // (not expected: a chunk of the group never published)
    if (split == 0 && threadIdx.x < kHeadDim) aa.out[(size_t)bh * kHeadDim + threadIdx.x] = __builtin_nanf("");
    return;
  }
  select_attend_head<kPaged, true>(aa, bh, split);
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

template <int R, bool kForced, bool kPaged, int kPasses>
static hipError_t launch_scan_passes(const Plan& p, const ScanArgs& sa, hipStream_t s) {
  const uint32_t shmem = (uint32_t)(R * p.chunk * sizeof(uint16_t));  // sorted slots, staged
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_kernel<R, kForced, kPaged, kPasses>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  launch_k(0, scan_kernel<R, kForced, kPaged, kPasses>, dim3(p.nch * p.B * p.Hkv), dim3(kScanThreads), shmem, s, sa.q,
           sa.codes, sa.kv_len, sa.Hq, sa.Hkv, sa.hkv_m, sa.nch, sa.nch_m, sa.xcd_map, sa.cap, sa.chunk, sa);
  return hipSuccess;
}

template <int R, bool kForced, bool kPaged>
static hipError_t launch_scan(const Plan& p, const ScanArgs& sa, hipStream_t s) {
  // (one instantiation per pass count: the pass loop is unrolled, and a block
  // fetches its kernel's code cold on every launch, so short chunks get a
  // kernel without the passes they never run)
  if (p.chunk > kSmallPasses * kScanThreads) return launch_scan_passes<R, kForced, kPaged, kScanPasses>(p, sa, s);
  if (p.chunk > 4 * kScanThreads) return launch_scan_passes<R, kForced, kPaged, kSmallPasses>(p, sa, s);
  if (p.chunk > kShortPasses * kScanThreads) return launch_scan_passes<R, kForced, kPaged, 4>(p, sa, s);
  if (p.chunk > kScanThreads) return launch_scan_passes<R, kForced, kPaged, kShortPasses>(p, sa, s);
  return launch_scan_passes<R, kForced, kPaged, 1>(p, sa, s);
}

template <int R>
static hipError_t launch_scan(const Plan& p, const ScanArgs& sa, bool forced, hipStream_t s) {
  if (sa.kv.table)
    return forced ? launch_scan<R, true, true>(p, sa, s) : launch_scan<R, false, true>(p, sa, s);
  return forced ? launch_scan<R, true, false>(p, sa, s) : launch_scan<R, false, false>(p, sa, s);
}

// Whether `grid` blocks of `kernel` (512 threads, `shmem` bytes of dynamic
// LDS) can all be resident on the current device at once.  (Cached: the last
// answer per kernel, LDS size and device.)
static bool all_resident(const void* kernel, int grid, uint32_t shmem) {
  struct Entry {
    const void* kernel;
    uint32_t shmem;
    int device, capacity;
  };
  static thread_local Entry cache[8];
  static thread_local int next = 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  for (const Entry& e : cache)
    if (e.kernel == kernel && e.shmem == shmem && e.device == dev) return grid <= e.capacity;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kScanThreads, shmem) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  cache[next] = Entry{kernel, shmem, dev, per_cu * cus};
  next = (next + 1) % 8;
  return grid <= per_cu * cus;
}

// The single-launch step, when every block fits on the device at once.
// Returns hipErrorNotReady (nothing launched) when it does not.
template <int R, bool kForced, bool kPaged>
static hipError_t launch_fused(const Plan& p, const ScanArgs& sa, const SelAttArgs& aa, const FusedSync& fs,
                               hipStream_t s) {
  const auto kernel = fused_decode_kernel<R, kForced, kPaged>;
  const size_t scan_lds = (size_t)R * p.chunk * sizeof(uint16_t);
  const uint32_t shmem = (uint32_t)(scan_lds > p.lds_select ? scan_lds : p.lds_select);
  const int grid = p.nch * p.B * p.Hkv;
  if (shmem > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
  }
  if (!all_resident(reinterpret_cast<const void*>(kernel), grid, shmem)) return hipErrorNotReady;
  launch_k(0, kernel, dim3(grid), dim3(kScanThreads), shmem, s, sa.q, sa.codes, sa.kv_len, sa.Hq, sa.Hkv, sa.hkv_m,
           sa.nch, sa.nch_m, sa.xcd_map, sa.cap, sa.chunk, sa, aa, fs);
  return hipSuccess;
}

template <int R>
static hipError_t launch_fused(const Plan& p, const ScanArgs& sa, const SelAttArgs& aa, const FusedSync& fs,
                               bool forced, hipStream_t s) {
  if (sa.kv.table)
    return forced ? launch_fused<R, true, true>(p, sa, aa, fs, s) : launch_fused<R, false, true>(p, sa, aa, fs, s);
  return forced ? launch_fused<R, true, false>(p, sa, aa, fs, s) : launch_fused<R, false, false>(p, sa, aa, fs, s);
}

hipError_t launch_decode(const Plan& p, const KvLayout& kv, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, uint8_t* codes, bool append, const Forced& f, const int32_t* kv_len,
                         float scale, float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, char* ws,
                         hipStream_t s) {
  uint16_t* ws_sorted = reinterpret_cast<uint16_t*>(ws + p.off_sorted);
  uint16_t* ws_rec = reinterpret_cast<uint16_t*>(ws + p.off_rec);
  float* ws_part = reinterpret_cast<float*>(ws + p.off_part);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + p.off_count);

  const bool forced = f.sink > 0 || f.recent > 0 || f.mask != nullptr;
  ScanArgs sa{q,       k,     codes,   kv_len, ws_sorted, ws_rec,   dist,          q_codes,
              counters, f.mask, p.Hq, p.Hkv, p.cap, p.chunk,   p.nch,    p.budget, append ? 1 : 0,
              f.sink, f.recent, f.mask_words, kv, div_magic(p.nch), div_magic(p.Hkv),
              (p.B * p.Hkv) % kXcds == 0 ? 1 : 0};
  SelAttArgs aa{q,      k,        v,       kv_len, ws_sorted, ws_rec,  ws_part, counters, sel_idx, out,
                scale * 1.4426950408889634f, p.Hq, p.Hkv, p.R, p.cap, p.budget, p.chunk, p.nch,
                p.pre_slots, p.splits, p.rows_per_split, p.bitmap_words,
                f.sink, f.recent, kv, div_magic(p.Hq)};
  launch_count() = 0;
  if (p.fused && launch_mode() == 1) {
    const FusedSync fs{reinterpret_cast<uint32_t*>(ws + p.off_sync),
                       reinterpret_cast<unsigned long long*>(ws + p.off_sync + kSyncFlagOffset)};
    hipError_t e = hipErrorInvalidValue;
    switch (p.R) {
      case 1: e = launch_fused<1>(p, sa, aa, fs, forced, s); break;
      case 2: e = launch_fused<2>(p, sa, aa, fs, forced, s); break;
      case 4: e = launch_fused<4>(p, sa, aa, fs, forced, s); break;
      case 8: e = launch_fused<8>(p, sa, aa, fs, forced, s); break;
    }
    if (e == hipSuccess) {
      launch_count() = 1;
      return hipGetLastError();
    }
    if (e != hipErrorNotReady) return e;
  }
  hipError_t es = hipErrorInvalidValue;
  switch (p.R) {
    case 1: es = launch_scan<1>(p, sa, forced, s); break;
    case 2: es = launch_scan<2>(p, sa, forced, s); break;
    case 4: es = launch_scan<4>(p, sa, forced, s); break;
    case 8: es = launch_scan<8>(p, sa, forced, s); break;
  }
  if (es != hipSuccess) return es;
  // In timing mode the select/attend kernel waits for the scan on the host, so
  // that its events bracket that kernel alone (not the dispatch gap after the scan).
  const ProfileEvents& pe = profile_events();
  if (pe.n >= 4) {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
  }
  const auto kernel = kv.table ? select_attend_kernel<true> : select_attend_kernel<false>;
  if (p.lds_select > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.lds_select);
    if (e != hipSuccess) return e;
  }
  launch_k(1, kernel, dim3(p.B * p.Hq, p.splits), dim3(kSAThreads), (uint32_t)p.lds_select, s, aa.q, aa.rec, aa.sorted,
           aa.kv_len, aa.Hq, aa.hq_m, aa.nch, aa.pre_slots, aa.chunk, aa);
  launch_count() = 2;
  return hipGetLastError();
}

}  // namespace adamas
