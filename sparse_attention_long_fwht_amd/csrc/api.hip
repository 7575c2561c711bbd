// api.hip -- the extern "C" entry points of libadamas.so (declared in
// include/adamas.h): argument checks, workspace sizing and kernel dispatch.
// Every host-checkable error is reported before anything is enqueued.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "adamas.h"
#include "plan.h"

using adamas::Plan;

namespace adamas {
static thread_local ProfileEvents t_profile{};
ProfileEvents& profile_events() { return t_profile; }
static thread_local int t_launch_mode = 0;
static thread_local int t_launch_count = 0;
int& launch_mode() { return t_launch_mode; }
int& launch_count() { return t_launch_count; }
}  // namespace adamas

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared shape checks.  need_q: num_q_heads participates.
adamas_status check_dims(const adamas_dims* d, bool need_q) {
  if (!d) return ADAMAS_ERR_INVALID_ARGUMENT;
  if (d->batch < 1 || d->num_kv_heads < 1 || d->capacity < 1 || d->head_dim < 1)
    return ADAMAS_ERR_INVALID_ARGUMENT;
  if (need_q) {
    if (d->num_q_heads < 1 || d->num_q_heads % d->num_kv_heads != 0) return ADAMAS_ERR_INVALID_ARGUMENT;
  }
  if (d->head_dim != ADAMAS_HEAD_DIM) return ADAMAS_ERR_UNSUPPORTED;
  if ((int64_t)d->capacity > adamas::kMaxCapacity) return ADAMAS_ERR_UNSUPPORTED;
  if ((int64_t)d->batch * d->num_kv_heads > 65535) return ADAMAS_ERR_UNSUPPORTED;
  if (need_q) {
    const int R = d->num_q_heads / d->num_kv_heads;
    if (R != 1 && R != 2 && R != 4 && R != 8) return ADAMAS_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->num_q_heads > 65535) return ADAMAS_ERR_UNSUPPORTED;
  }
  return ADAMAS_OK;
}

adamas::KvLayout contiguous_layout(const adamas_dims* d) {
  return adamas::KvLayout{nullptr, 0, 0, 0, d->num_kv_heads, d->capacity, adamas::div_magic(d->num_kv_heads)};
}

// Checks a page description against the dims (after check_dims) and builds the layout.
adamas_status paged_layout(const adamas_dims* d, const adamas_pages* pg, adamas::KvLayout* kv) {
  if (!pg || !pg->block_table || !aligned(pg->block_table, 4)) return ADAMAS_ERR_INVALID_ARGUMENT;
  const int32_t ps = pg->page_size;
  if (ps < 1 || ps > (1 << 20) || (ps & (ps - 1)) != 0 || pg->max_pages < 1 || pg->num_pages < 1)
    return ADAMAS_ERR_INVALID_ARGUMENT;
  if ((int64_t)pg->max_pages * ps < d->capacity) return ADAMAS_ERR_INVALID_ARGUMENT;
  if ((int64_t)d->batch * pg->max_pages > ((int64_t)1 << 31)) return ADAMAS_ERR_UNSUPPORTED;
  *kv = adamas::KvLayout{pg->block_table, pg->max_pages, __builtin_ctz((unsigned)ps), pg->num_pages,
                         d->num_kv_heads, d->capacity, adamas::div_magic(d->num_kv_heads)};
  return ADAMAS_OK;
}

}  // namespace

extern "C" {

const char* adamas_status_string(adamas_status s) {
  switch (s) {
    case ADAMAS_OK: return "ok";
    case ADAMAS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case ADAMAS_ERR_UNSUPPORTED: return "unsupported shape or size";
    case ADAMAS_ERR_WORKSPACE: return "workspace missing or too small";
    case ADAMAS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t adamas_abi_version(void) { return ADAMAS_ABI_VERSION; }

adamas_status adamas_decode_launch_mode(int32_t mode) {
  if (mode != 0 && mode != 1) return ADAMAS_ERR_INVALID_ARGUMENT;
  adamas::launch_mode() = mode;
  return ADAMAS_OK;
}

int32_t adamas_last_launch_count(void) { return adamas::launch_count(); }

adamas_status adamas_profile_events(void* const* events, int32_t n_events) {
  if (n_events < 0 || n_events > adamas::kMaxProfileEvents || (!events && n_events > 0))
    return ADAMAS_ERR_INVALID_ARGUMENT;
  adamas::ProfileEvents& pe = adamas::profile_events();
  pe.n = events ? n_events : 0;
  for (int i = 0; i < pe.n; ++i) pe.ev[i] = static_cast<hipEvent_t>(events[i]);
  return ADAMAS_OK;
}

}  // extern "C"

namespace {

adamas_status encode_common(const adamas_dims* d, const adamas_pages* pages, const void* k, const int32_t* start,
                            const int32_t* end, uint8_t* codes, void* stream, int32_t max_rows = 0) {
  adamas_status st = check_dims(d, false);
  if (st != ADAMAS_OK) return st;
  if (max_rows < 0) return ADAMAS_ERR_INVALID_ARGUMENT;
  if (!k || !end || !codes) return ADAMAS_ERR_INVALID_ARGUMENT;
  if (!aligned(k, 16) || !aligned(codes, 16) || !aligned(end, 4) || (start && !aligned(start, 4)))
    return ADAMAS_ERR_INVALID_ARGUMENT;
  adamas::KvLayout kv = contiguous_layout(d);
  if (pages && (st = paged_layout(d, pages, &kv)) != ADAMAS_OK) return st;
  hipError_t e = adamas::launch_encode_keys(d->batch, kv, static_cast<const uint16_t*>(k), start, end, codes,
                                            static_cast<hipStream_t>(stream), max_rows);
  return e == hipSuccess ? ADAMAS_OK : ADAMAS_ERR_HIP;
}

}  // namespace

extern "C" {

adamas_status adamas_encode_keys(const adamas_dims* d, const void* k, const int32_t* start, const int32_t* end,
                                 uint8_t* codes, void* stream) {
  return encode_common(d, nullptr, k, start, end, codes, stream);
}

adamas_status adamas_paged_encode_keys(const adamas_dims* d, const adamas_pages* pages, const void* k_pool,
                                       const int32_t* start, const int32_t* end, uint8_t* codes_pool,
                                       void* stream) {
  if (!pages) return ADAMAS_ERR_INVALID_ARGUMENT;
  return encode_common(d, pages, k_pool, start, end, codes_pool, stream);
}

adamas_status adamas_encode_keys_bounded(const adamas_dims* d, const void* k, const int32_t* start,
                                         const int32_t* end, int32_t max_rows, uint8_t* codes, void* stream) {
  if (max_rows < 1) return ADAMAS_ERR_INVALID_ARGUMENT;
  return encode_common(d, nullptr, k, start, end, codes, stream, max_rows);
}

adamas_status adamas_paged_encode_keys_bounded(const adamas_dims* d, const adamas_pages* pages,
                                               const void* k_pool, const int32_t* start, const int32_t* end,
                                               int32_t max_rows, uint8_t* codes_pool, void* stream) {
  if (!pages || max_rows < 1) return ADAMAS_ERR_INVALID_ARGUMENT;
  return encode_common(d, pages, k_pool, start, end, codes_pool, stream, max_rows);
}

size_t adamas_decode_workspace_size(const adamas_dims* d, int32_t budget) {
  if (check_dims(d, true) != ADAMAS_OK || budget < 1) return 0;
  const Plan p = adamas::make_plan(d->batch, d->num_q_heads, d->num_kv_heads, d->capacity, budget, false);
  return p.supported ? p.total : 0;
}

}  // extern "C"

namespace {

adamas_status decode_common(const adamas_dims* d, const adamas_pages* pages, const void* q, const void* k,
                            const void* v, uint8_t* codes, bool append, const adamas_forced* forced,
                            const int32_t* kv_len, int32_t budget, float scale, float* out, int32_t* sel_idx,
                            uint16_t* dist, uint8_t* q_codes, void* workspace, size_t workspace_bytes,
                            void* stream) {
  adamas_status st = check_dims(d, true);
  if (st != ADAMAS_OK) return st;
  if (!q || !k || !v || !codes || !kv_len || !out || budget < 1) return ADAMAS_ERR_INVALID_ARGUMENT;
  adamas::KvLayout kv = contiguous_layout(d);
  if (pages && (st = paged_layout(d, pages, &kv)) != ADAMAS_OK) return st;
  adamas::Forced f{0, 0, nullptr, 0};
  if (forced) {
    if (forced->sink < 0 || forced->recent < 0 || (int64_t)forced->sink + forced->recent > budget)
      return ADAMAS_ERR_INVALID_ARGUMENT;
    if (forced->mask && (!aligned(forced->mask, 4) || (int64_t)forced->mask_words * 32 < d->capacity))
      return ADAMAS_ERR_INVALID_ARGUMENT;
    f = adamas::Forced{forced->sink, forced->recent, forced->mask, forced->mask ? forced->mask_words : 0};
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(codes, 16) || !aligned(kv_len, 4) ||
      !aligned(out, 4) || (sel_idx && !aligned(sel_idx, 4)) || (dist && !aligned(dist, 2)) ||
      (q_codes && !aligned(q_codes, 4)))
    return ADAMAS_ERR_INVALID_ARGUMENT;
  const Plan p = adamas::make_plan(d->batch, d->num_q_heads, d->num_kv_heads, d->capacity, budget, false);
  if (!p.supported) return ADAMAS_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)) return ADAMAS_ERR_WORKSPACE;
  hipError_t e = adamas::launch_decode(p, kv, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                       static_cast<const uint16_t*>(v), codes, append, f, kv_len, scale, out, sel_idx,
                                       dist, q_codes, static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADAMAS_OK : ADAMAS_ERR_HIP;
}

}  // namespace

extern "C" {

adamas_status adamas_decode_step(const adamas_dims* d, const void* q, const void* k, const void* v,
                                 const uint8_t* codes, const int32_t* kv_len, int32_t budget, float scale,
                                 float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  // codes are only read on this path
  return decode_common(d, nullptr, q, k, v, const_cast<uint8_t*>(codes), false, nullptr, kv_len, budget, scale, out,
                       sel_idx, dist, q_codes, workspace, workspace_bytes, stream);
}

adamas_status adamas_append_decode_step(const adamas_dims* d, const void* q, const void* k, const void* v,
                                        uint8_t* codes, const int32_t* kv_len, int32_t budget, float scale,
                                        float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(d, nullptr, q, k, v, codes, true, nullptr, kv_len, budget, scale, out, sel_idx, dist,
                       q_codes, workspace, workspace_bytes, stream);
}

adamas_status adamas_forced_decode_step(const adamas_dims* d, const adamas_forced* forced, int32_t append,
                                        const void* q, const void* k, const void* v, uint8_t* codes,
                                        const int32_t* kv_len, int32_t budget, float scale, float* out,
                                        int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (!forced || (append != 0 && append != 1)) return ADAMAS_ERR_INVALID_ARGUMENT;
  return decode_common(d, nullptr, q, k, v, codes, append != 0, forced, kv_len, budget, scale, out, sel_idx, dist,
                       q_codes, workspace, workspace_bytes, stream);
}

adamas_status adamas_paged_decode_step(const adamas_dims* d, const adamas_pages* pages, const adamas_forced* forced,
                                       int32_t append, const void* q, const void* k_pool, const void* v_pool,
                                       uint8_t* codes_pool, const int32_t* kv_len, int32_t budget, float scale,
                                       float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  if (!pages || (append != 0 && append != 1)) return ADAMAS_ERR_INVALID_ARGUMENT;
  return decode_common(d, pages, q, k_pool, v_pool, codes_pool, append != 0, forced, kv_len, budget, scale, out,
                       sel_idx, dist, q_codes, workspace, workspace_bytes, stream);
}

size_t dense_decode_workspace_size(const adamas_dims* d) {
  if (check_dims(d, true) != ADAMAS_OK) return 0;
  return adamas::make_plan(d->batch, d->num_q_heads, d->num_kv_heads, d->capacity, 1, true).total;
}

}  // extern "C"

namespace {

adamas_status dense_common(const adamas_dims* d, const adamas_pages* pages, const void* q, const void* k,
                           const void* v, const int32_t* kv_len, float scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  adamas_status st = check_dims(d, true);
  if (st != ADAMAS_OK) return st;
  adamas::KvLayout kv = contiguous_layout(d);
  if (pages && (st = paged_layout(d, pages, &kv)) != ADAMAS_OK) return st;
  if (!q || !k || !v || !kv_len || !out) return ADAMAS_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(kv_len, 4) || !aligned(out, 4))
    return ADAMAS_ERR_INVALID_ARGUMENT;
  const Plan p = adamas::make_plan(d->batch, d->num_q_heads, d->num_kv_heads, d->capacity, 1, true);
  if (!workspace || workspace_bytes < p.total || !aligned(workspace, 256)) return ADAMAS_ERR_WORKSPACE;
  hipError_t e = adamas::launch_dense(p, kv, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), kv_len, scale, out,
                                      static_cast<char*>(workspace), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ADAMAS_OK : ADAMAS_ERR_HIP;
}

}  // namespace

extern "C" {

adamas_status dense_decode_attention(const adamas_dims* d, const void* q, const void* k, const void* v,
                                     const int32_t* kv_len, float scale, float* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return dense_common(d, nullptr, q, k, v, kv_len, scale, out, workspace, workspace_bytes, stream);
}

adamas_status dense_paged_decode_attention(const adamas_dims* d, const adamas_pages* pages, const void* q,
                                           const void* k_pool, const void* v_pool, const int32_t* kv_len,
                                           float scale, float* out, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (!pages) return ADAMAS_ERR_INVALID_ARGUMENT;
  return dense_common(d, pages, q, k_pool, v_pool, kv_len, scale, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The decode step without a caller workspace (adamas_decode_step_noalloc).
// Its scratch is this file-scope device array: each GPU the library runs on
// holds its own copy, allocated with the code object and kept until the
// process ends.  In host code `scratch` names a host-side stand-in, so its
// device address is taken once per device with hipGetSymbolAddress (with
// that device current) and only that address is passed to kernels.
// ---------------------------------------------------------------------------
namespace {

__device__ __align__(256) char scratch[ADAMAS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address (nullptr on a HIP error).
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

adamas_status adamas_decode_step_noalloc(const adamas_dims* d, const void* q, const void* k, const void* v,
                                         const uint8_t* codes, const int32_t* kv_len, int32_t budget, float scale,
                                         float* out, int32_t* sel_idx, uint16_t* dist, uint8_t* q_codes,
                                         void* stream) {
  // the checks of adamas_decode_step, then the size against the static area,
  // all before any HIP call
  adamas_status st = check_dims(d, true);
  if (st != ADAMAS_OK) return st;
  if (!q || !k || !v || !codes || !kv_len || !out || budget < 1) return ADAMAS_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(codes, 16) || !aligned(kv_len, 4) ||
      !aligned(out, 4) || (sel_idx && !aligned(sel_idx, 4)) || (dist && !aligned(dist, 2)) ||
      (q_codes && !aligned(q_codes, 4)))
    return ADAMAS_ERR_INVALID_ARGUMENT;
  const Plan p = adamas::make_plan(d->batch, d->num_q_heads, d->num_kv_heads, d->capacity, budget, false);
  if (!p.supported || p.total > (size_t)ADAMAS_NOALLOC_SCRATCH_BYTES) return ADAMAS_ERR_UNSUPPORTED;
  void* ws = scratch_for_current_device();
  if (!ws) return ADAMAS_ERR_HIP;
  return decode_common(d, nullptr, q, k, v, const_cast<uint8_t*>(codes), false, nullptr, kv_len, budget, scale,
                       out, sel_idx, dist, q_codes, ws, (size_t)ADAMAS_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
