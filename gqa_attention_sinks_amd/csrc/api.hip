// C ABI of libsinkattn: argument validation on the host, then kernel launches
// on the caller's stream.  Declarations and the contract of every entry point
// are in include/sinkattn.h.

#include <math.h>
#include <stdint.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "kernel_args.hpp"
#include "sinkattn.h"

namespace sinkattn {
int prefill_rows_per_tile(int32_t window, int32_t group);
}

namespace {

thread_local std::string g_last_error;

sinkattn_status fail(sinkattn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sinkattn_status fail(sinkattn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

sinkattn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SINKATTN_OK;
  return fail(SINKATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

sinkattn_status check_heads(int32_t batch, int32_t hq, int32_t hkv, int32_t head_dim, float sm_scale,
                            int32_t window) {
  REQUIRE(batch >= 1, SINKATTN_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  REQUIRE(hq >= 1 && hkv >= 1, SINKATTN_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", hq, hkv);
  REQUIRE(hq % hkv == 0, SINKATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", hq, hkv);
  REQUIRE(head_dim == SINKATTN_HEAD_DIM, SINKATTN_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", head_dim);
  REQUIRE(hq / hkv <= 16, SINKATTN_ERR_UNSUPPORTED, "Hq/Hkv = %d unsupported (at most 16)", hq / hkv);
  REQUIRE(isfinite(sm_scale) && sm_scale > 0.f, SINKATTN_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  REQUIRE(window >= 0, SINKATTN_ERR_INVALID_ARG, "window must be >= 0 (got %d)", window);
  return SINKATTN_OK;
}

sinkattn_status check_kv(const sinkattn_kv* kv, bool need_paged) {
  REQUIRE(kv != nullptr, SINKATTN_ERR_INVALID_ARG, "kv descriptor is NULL");
  REQUIRE(kv->k != nullptr && kv->v != nullptr, SINKATTN_ERR_INVALID_ARG, "kv->k and kv->v are required");
  REQUIRE(kv->kv_indptr != nullptr, SINKATTN_ERR_INVALID_ARG, "kv->kv_indptr is required");
  REQUIRE(kv->paged == 0 || kv->paged == 1, SINKATTN_ERR_INVALID_ARG, "kv->paged must be 0 or 1");
  if (need_paged) REQUIRE(kv->paged == 1, SINKATTN_ERR_INVALID_ARG, "decode needs a paged KV cache");
  if (kv->paged) {
    REQUIRE(kv->page_indices != nullptr && kv->kv_len != nullptr, SINKATTN_ERR_INVALID_ARG,
            "paged KV needs page_indices and kv_len");
    REQUIRE(kv->page_size == SINKATTN_PAGE_SIZE, SINKATTN_ERR_UNSUPPORTED,
            "page_size %d unsupported (only 16)", kv->page_size);
  }
  return SINKATTN_OK;
}

// Partials of sinkattn_decode_paged_noalloc: a file-scope device array, one
// copy per GPU at its own address.  Host code never passes `scratch` itself
// to a kernel (in host code the name is only a stand-in for the symbol): it
// uses the device address that hipGetSymbolAddress returns for the current
// device, looked up on the first call there and kept per device.
__device__ __align__(256) unsigned char scratch[SINKATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

sinkattn_status scratch_on_current_device(void** ptr) {
  int dev = -1;
  sinkattn_status st = hip_status(hipGetDevice(&dev), "hipGetDevice");
  if (st != SINKATTN_OK) return st;
  REQUIRE(dev >= 0 && dev < kMaxDevices, SINKATTN_ERR_UNSUPPORTED, "device %d: at most %d devices", dev,
          kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (st != SINKATTN_OK) return st;
    REQUIRE(p != nullptr, SINKATTN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return SINKATTN_OK;
}

// The longest-first order of a decode launch's requests (ties by index: the
// order the kernels' own ranking gives), from the caller's host copy of
// kv_len, under the same conditions as that ranking; otherwise the kernels
// rank the batch (or take the requests in order) themselves.  Any order gives
// the same results, so a stale or wrong host copy only costs time.
void plan_decode_order(const sinkattn_kv* kv, int32_t batch, int32_t window, sinkattn::DecodeArgs* d) {
  if (kv->kv_len_host == nullptr || batch < 2 || batch > sinkattn::kPlanMaxBatch ||
      (window > 0 && window <= sinkattn::kPlanMinWindow))
    return;
  const int32_t* len = kv->kv_len_host;
  int32_t idx[sinkattn::kPlanMaxBatch];
  for (int32_t b = 0; b < batch; ++b) idx[b] = b;
  std::stable_sort(idx, idx + batch, [len](int32_t x, int32_t y) { return len[x] > len[y]; });
  for (int32_t r = 0; r < batch; ++r) d->order[r] = static_cast<uint16_t>(idx[r]);
  d->planned = 1;
}

// The (request, tile) of every prefill tile slot, in the order the kernel's
// own scan gives (see kPrefillRankMaxTiles), from the caller's host copy of
// qo_indptr (and of kv_len when the kernel would rank tiles by their key
// counts).  The set of tiles follows qo_indptr alone; their order only sets
// when each runs, so any copy of kv_len gives the same results.  Without key
// counts on the host (contiguous KV), a launch of several requests that the
// kernel would rank keeps the kernel's scan.
bool plan_prefill_tiles(const sinkattn_kv* kv, const int32_t* qo_host, int32_t batch, int32_t window, int bm,
                        long slots, const sinkattn::PrefillArgs& a, sinkattn::PrefillPlan* plan) {
  using sinkattn::kPrefillPlanMax;
  constexpr int kKeys = sinkattn::kPrefillTileKeys;
  if (slots < 1 || slots > kPrefillPlanMax || batch > 65536) return false;
  const bool may_rank = slots <= sinkattn::kPrefillRankMaxTiles && (window == 0 || window > sinkattn::kPlanMinWindow);
  const int32_t* nk_host = kv->paged ? kv->kv_len_host : nullptr;
  if (may_rank && nk_host == nullptr && batch > 1) return false;   // one request: nothing to rank
  auto n_q = [&](int32_t b) { return qo_host[b + 1] - qo_host[b]; };
  auto n_tiles = [&](int32_t b) { return (a.skip_single_rows && n_q(b) == 1) ? 0 : (n_q(b) + bm - 1) / bm; };
  for (int32_t b = 0; b < batch; ++b)
    if (n_q(b) > 65535 * bm) return false;   // tile numbers must fit 16 bits
  bool uniform = true;                 // every request shaped like request 0 (single rows included)
  if (may_rank)
    for (int32_t b = 1; b < batch && uniform; ++b) uniform = n_q(b) == n_q(0) && nk_host[b] == nk_host[0];
  long r = 0;
  if (may_rank && !uniform) {
    // tiles request by request, then stably by decreasing key count
    uint32_t tile_of[kPrefillPlanMax];
    int64_t work[kPrefillPlanMax];
    int32_t idx[kPrefillPlanMax];
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t shift = (int64_t)nk_host[b] - n_q(b);
      for (int32_t t = 0; t < n_tiles(b); ++t, ++r) {
        const int64_t t0 = (int64_t)t * bm;
        const int64_t t_last = std::min<int64_t>(t0 + bm, n_q(b)) - 1;
        const int64_t lo_first = window > 0 ? std::max<int64_t>(0, shift + t0 - window + 1) : 0;
        const int64_t k_first = lo_first / kKeys * kKeys;
        work[r] = (shift + t_last + 1 - k_first + kKeys - 1) / kKeys;
        tile_of[r] = (uint32_t)b << 16 | (uint32_t)t;
        idx[r] = (int32_t)r;
      }
    }
    std::stable_sort(idx, idx + r, [&work](int32_t x, int32_t y) { return work[x] > work[y]; });
    for (long i = 0; i < r; ++i) plan->slot[i] = tile_of[idx[i]];
  } else {
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t nt = n_tiles(b);
      for (int32_t s = 0; s < nt; ++s) plan->slot[r++] = (uint32_t)b << 16 | (uint32_t)(nt - 1 - s);
    }
  }
  return r == slots;   // (always: slots counts the same tiles)
}

}  // namespace

extern "C" {

sinkattn_status sinkattn_prefill(const void* q, const int32_t* qo_indptr, const sinkattn_kv* kv,
                                 const float* sinks, void* out, float* lse, int32_t batch,
                                 int32_t total_q, int32_t num_qo_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float sm_scale, int32_t window,
                                 const int32_t* qo_indptr_host, void* stream) {
  REQUIRE(q != nullptr && qo_indptr != nullptr && out != nullptr, SINKATTN_ERR_INVALID_ARG,
          "q, qo_indptr and out are required");
  sinkattn_status st = check_heads(batch, num_qo_heads, num_kv_heads, head_dim, sm_scale, window);
  if (st != SINKATTN_OK) return st;
  if ((st = check_kv(kv, false)) != SINKATTN_OK) return st;
  REQUIRE(total_q >= batch, SINKATTN_ERR_INVALID_ARG, "total_q (%d) must be >= batch (%d): every request has a query row",
          total_q, batch);

  const int bm = sinkattn::prefill_rows_per_tile(window, num_qo_heads / num_kv_heads);
  sinkattn::PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.qo_indptr = qo_indptr;
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  a.kv_indptr = kv->kv_indptr;
  a.page_indices = kv->page_indices;
  a.kv_len = kv->kv_len;
  a.sinks = sinks;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.batch = batch;
  a.num_qo_heads = num_qo_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_qo_heads / num_kv_heads;
  a.window = window;
  a.paged = kv->paged;
  // single-row requests (decode rows of a mixed batch) go to the decode kernel when paged
  a.skip_single_rows = kv->paged;
  long slots = (long)total_q / bm + batch;   // >= sum over requests of ceil(n_q / bm)
  bool any_single = true;                    // a request with one row may exist
  if (qo_indptr_host != nullptr) {           // exact plan from the host copy
    slots = 0;
    any_single = false;
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t n = (int64_t)qo_indptr_host[b + 1] - qo_indptr_host[b];
      REQUIRE(n >= 1, SINKATTN_ERR_INVALID_ARG, "request %d has no query row", b);
      if (kv->paged && n == 1) {
        any_single = true;
        continue;
      }
      slots += (n + bm - 1) / bm;
    }
    REQUIRE(qo_indptr_host[batch] == total_q, SINKATTN_ERR_INVALID_ARG,
            "qo_indptr_host[batch] (%d) != total_q (%d)", qo_indptr_host[batch], total_q);
  }
  REQUIRE(slots * num_qo_heads < (1L << 31), SINKATTN_ERR_UNSUPPORTED, "launch too large");
  a.num_slots = (int32_t)slots;
  sinkattn::PrefillPlan plan;
  const bool planned =
      qo_indptr_host != nullptr && plan_prefill_tiles(kv, qo_indptr_host, batch, window, bm, slots, a, &plan);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (slots > 0 &&
      (st = hip_status(sinkattn::launch_prefill(a, planned ? &plan : nullptr, s), "prefill launch")) != SINKATTN_OK)
    return st;
  if (kv->paged && any_single) {
    sinkattn::DecodeArgs d{};
    d.q = a.q;
    d.k_pool = a.k;
    d.v_pool = a.v;
    d.page_indptr = kv->kv_indptr;
    d.page_indices = kv->page_indices;
    d.kv_len = kv->kv_len;
    d.qo_indptr = qo_indptr;
    d.sinks = sinks;
    d.out = a.out;
    d.lse = lse;
    d.scale_log2 = a.scale_log2;
    d.batch = batch;
    d.num_qo_heads = num_qo_heads;
    d.num_kv_heads = num_kv_heads;
    d.group = a.group;
    d.num_splits = 1;
    d.window = window;
    plan_decode_order(kv, batch, window, &d);
    if ((st = hip_status(sinkattn::launch_decode(d, s), "decode launch")) != SINKATTN_OK) return st;
  }
  return SINKATTN_OK;
}

sinkattn_status sinkattn_decode_paged(const void* q, const sinkattn_kv* kv, const float* sinks,
                                      int32_t num_splits, void* out, float* o_part,
                                      float* lse_part, float* lse, int32_t batch,
                                      int32_t num_qo_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float sm_scale, int32_t window,
                                      void* stream) {
  REQUIRE(q != nullptr, SINKATTN_ERR_INVALID_ARG, "q is required");
  sinkattn_status st = check_heads(batch, num_qo_heads, num_kv_heads, head_dim, sm_scale, window);
  if (st != SINKATTN_OK) return st;
  if ((st = check_kv(kv, true)) != SINKATTN_OK) return st;
  REQUIRE(num_splits >= 1 && num_splits <= SINKATTN_MAX_SPLITS, SINKATTN_ERR_INVALID_ARG,
          "num_splits must be in [1, %d] (got %d)", SINKATTN_MAX_SPLITS, num_splits);
  if (num_splits == 1) {
    REQUIRE(out != nullptr, SINKATTN_ERR_INVALID_ARG, "num_splits == 1 needs out");
  } else {
    REQUIRE(o_part != nullptr && lse_part != nullptr, SINKATTN_ERR_INVALID_ARG,
            "num_splits > 1 needs o_part and lse_part");
  }
  sinkattn::DecodeArgs d{};
  d.q = static_cast<const uint16_t*>(q);
  d.k_pool = static_cast<const uint16_t*>(kv->k);
  d.v_pool = static_cast<const uint16_t*>(kv->v);
  d.page_indptr = kv->kv_indptr;
  d.page_indices = kv->page_indices;
  d.kv_len = kv->kv_len;
  d.qo_indptr = nullptr;
  d.sinks = sinks;
  d.out = static_cast<uint16_t*>(out);
  d.lse = lse;
  d.o_part = o_part;
  d.lse_part = lse_part;
  d.scale_log2 = sm_scale * 1.4426950408889634f;
  d.batch = batch;
  d.num_qo_heads = num_qo_heads;
  d.num_kv_heads = num_kv_heads;
  d.group = num_qo_heads / num_kv_heads;
  d.num_splits = num_splits;
  d.window = window;
  REQUIRE((long)batch * num_kv_heads * num_splits < (1L << 31), SINKATTN_ERR_UNSUPPORTED, "launch too large");
  plan_decode_order(kv, batch, window, &d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(sinkattn::launch_decode(d, s), "decode launch")) != SINKATTN_OK) return st;
  if (num_splits > 1 && out != nullptr) {
    sinkattn::MergeArgs m{o_part, lse_part, static_cast<uint16_t*>(out), lse, batch, num_qo_heads, num_splits};
    if ((st = hip_status(sinkattn::launch_merge(m, s), "merge launch")) != SINKATTN_OK) return st;
  }
  return SINKATTN_OK;
}

sinkattn_status sinkattn_decode_paged_noalloc(const void* q, const sinkattn_kv* kv, const float* sinks,
                                              int32_t num_splits, void* out, float* lse, int32_t batch,
                                              int32_t num_qo_heads, int32_t num_kv_heads,
                                              int32_t head_dim, float sm_scale, int32_t window,
                                              void* stream) {
  REQUIRE(q != nullptr && out != nullptr, SINKATTN_ERR_INVALID_ARG, "q and out are required");
  sinkattn_status st = check_heads(batch, num_qo_heads, num_kv_heads, head_dim, sm_scale, window);
  if (st != SINKATTN_OK) return st;
  if ((st = check_kv(kv, true)) != SINKATTN_OK) return st;
  REQUIRE(num_splits >= 1 && num_splits <= SINKATTN_MAX_SPLITS, SINKATTN_ERR_INVALID_ARG,
          "num_splits must be in [1, %d] (got %d)", SINKATTN_MAX_SPLITS, num_splits);
  if (num_splits == 1)   // nothing to merge: no partials, no scratch
    return sinkattn_decode_paged(q, kv, sinks, 1, out, nullptr, nullptr, lse, batch, num_qo_heads, num_kv_heads,
                                 head_dim, sm_scale, window, stream);
  // o_part [batch, Hq, S, 64] then lse_part [batch, Hq, S], each 256-byte aligned
  const size_t parts = (size_t)batch * num_qo_heads * num_splits;
  const size_t o_bytes = (parts * SINKATTN_HEAD_DIM * sizeof(float) + 255) & ~(size_t)255;
  const size_t need = o_bytes + parts * sizeof(float);
  REQUIRE(need <= SINKATTN_NOALLOC_SCRATCH_BYTES, SINKATTN_ERR_INVALID_ARG,
          "batch %d x %d heads x %d splits needs %zu bytes of partials, more than the %u-byte scratch "
          "array; use sinkattn_decode_paged with caller-owned partials", batch, num_qo_heads, num_splits, need,
          (unsigned)SINKATTN_NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  if ((st = scratch_on_current_device(&base)) != SINKATTN_OK) return st;
  float* o_part = static_cast<float*>(base);
  float* lse_part = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + o_bytes);
  return sinkattn_decode_paged(q, kv, sinks, num_splits, out, o_part, lse_part, lse, batch, num_qo_heads,
                               num_kv_heads, head_dim, sm_scale, window, stream);
}

int64_t sinkattn_decode_balanced_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t num_segments) {
  if (batch < 1 || num_qo_heads < 1 || num_segments < 1) return -1;
  const int64_t slots = (int64_t)num_segments + batch;
  const int64_t plan = ((int64_t)(3 * batch + 1) * 4 + 255) & ~(int64_t)255;
  const int64_t lse = (slots * num_qo_heads * 4 + 255) & ~(int64_t)255;
  return plan + lse + slots * num_qo_heads * SINKATTN_HEAD_DIM * 4;
}

int32_t sinkattn_pick_num_segments(int32_t num_kv_heads) {
  if (num_kv_heads < 1) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int32_t n = (cus * sinkattn::kBalancedWavesPerSimd + num_kv_heads - 1) / num_kv_heads;
  return n > 1 ? n : 1;
}

sinkattn_status sinkattn_balanced_segments(const int32_t* kv_len_host, int32_t batch, int32_t window,
                                           int32_t num_segments, int32_t* segs_host) {
  REQUIRE(kv_len_host != nullptr && segs_host != nullptr, SINKATTN_ERR_INVALID_ARG,
          "kv_len_host and segs_host are required");
  REQUIRE(batch >= 0, SINKATTN_ERR_INVALID_ARG, "batch must be >= 0");
  REQUIRE(window >= 0, SINKATTN_ERR_INVALID_ARG, "window must be >= 0");
  REQUIRE(num_segments >= 1 && num_segments <= 65536, SINKATTN_ERR_INVALID_ARG,
          "num_segments must be in [1, 65536]");
  int64_t total = 0;
  for (int32_t b = 0; b < batch; ++b) {
    REQUIRE(kv_len_host[b] >= 0, SINKATTN_ERR_INVALID_ARG, "kv_len[%d] < 0", b);
    const int64_t n_k = kv_len_host[b];
    const int64_t lo = window > 0 ? (n_k - window > 0 ? n_k - window : 0) : 0;
    total += n_k > 0 ? (n_k + SINKATTN_PAGE_SIZE - 1) / SINKATTN_PAGE_SIZE - lo / SINKATTN_PAGE_SIZE : 0;
  }
  int64_t pos = 0;   // list position of the request's first live page
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n_k = kv_len_host[b];
    const int64_t lo = window > 0 ? (n_k - window > 0 ? n_k - window : 0) : 0;
    const int64_t n = n_k > 0 ? (n_k + SINKATTN_PAGE_SIZE - 1) / SINKATTN_PAGE_SIZE - lo / SINKATTN_PAGE_SIZE : 0;
    // list position f lies in segment floor(((f + 1) N - 1) / T)
    segs_host[2 * b] = n > 0 ? (int32_t)(((pos + 1) * num_segments - 1) / total) : -1;
    segs_host[2 * b + 1] = n > 0 ? (int32_t)(((pos + n) * num_segments - 1) / total) : -1;
    pos += n;
  }
  return SINKATTN_OK;
}

}  // extern "C"

namespace {

// Arguments of the balanced decode's launches, checked; `need_kv`: the
// pieces launch (the merge reads only the workspace, sinks and outputs).
sinkattn_status balanced_args(const void* q, const sinkattn_kv* kv, const float* sinks, int32_t num_segments,
                              const void* workspace, int64_t workspace_bytes, void* out, float* lse,
                              int32_t batch, int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                              float sm_scale, int32_t window, bool need_kv, sinkattn::BalancedArgs* a) {
  REQUIRE(out != nullptr && workspace != nullptr, SINKATTN_ERR_INVALID_ARG, "out and workspace are required");
  sinkattn_status st = check_heads(batch, num_qo_heads, num_kv_heads, head_dim, sm_scale, window);
  if (st != SINKATTN_OK) return st;
  if (need_kv) {
    REQUIRE(q != nullptr, SINKATTN_ERR_INVALID_ARG, "q is required");
    if ((st = check_kv(kv, true)) != SINKATTN_OK) return st;
  }
  REQUIRE(batch <= SINKATTN_MAX_BALANCED_BATCH, SINKATTN_ERR_UNSUPPORTED,
          "batch %d above %d: use sinkattn_decode_paged", batch, SINKATTN_MAX_BALANCED_BATCH);
  REQUIRE(num_segments >= 1 && num_segments <= 65536, SINKATTN_ERR_INVALID_ARG,
          "num_segments must be in [1, 65536] (got %d)", num_segments);
  REQUIRE(((uintptr_t)workspace & 15) == 0, SINKATTN_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const int64_t need = sinkattn_decode_balanced_workspace_bytes(batch, num_qo_heads, num_segments);
  REQUIRE(workspace_bytes >= need, SINKATTN_ERR_INVALID_ARG, "workspace of %lld bytes, %lld needed",
          (long long)workspace_bytes, (long long)need);
  REQUIRE((long)num_segments * num_kv_heads < (1L << 31), SINKATTN_ERR_UNSUPPORTED, "launch too large");
  const int64_t slots = (int64_t)num_segments + batch;
  unsigned char* ws = static_cast<unsigned char*>(const_cast<void*>(workspace));
  const int64_t plan_bytes = ((int64_t)(3 * batch + 1) * 4 + 255) & ~(int64_t)255;
  const int64_t lse_bytes = (slots * num_qo_heads * 4 + 255) & ~(int64_t)255;
  *a = sinkattn::BalancedArgs{};
  a->q = static_cast<const uint16_t*>(q);
  if (need_kv) {
    a->k_pool = static_cast<const uint16_t*>(kv->k);
    a->v_pool = static_cast<const uint16_t*>(kv->v);
    a->page_indptr = kv->kv_indptr;
    a->page_indices = kv->page_indices;
    a->kv_len = kv->kv_len;
  }
  a->sinks = sinks;
  a->out = static_cast<uint16_t*>(out);
  a->lse = lse;
  a->ws_plan = reinterpret_cast<int32_t*>(ws);
  a->ws_seg = a->ws_plan + batch + 1;
  a->ws_lse = reinterpret_cast<float*>(ws + plan_bytes);
  a->ws_o = reinterpret_cast<float*>(ws + plan_bytes + lse_bytes);
  a->scale_log2 = sm_scale * 1.4426950408889634f;
  a->batch = batch;
  a->num_qo_heads = num_qo_heads;
  a->num_kv_heads = num_kv_heads;
  a->group = num_qo_heads / num_kv_heads;
  a->window = window;
  a->num_segments = num_segments;
  return SINKATTN_OK;
}

}  // namespace

extern "C" {

sinkattn_status sinkattn_decode_paged_balanced_pieces(const void* q, const sinkattn_kv* kv, const float* sinks,
                                                      int32_t num_segments, void* workspace,
                                                      int64_t workspace_bytes, void* out, float* lse,
                                                      int32_t batch, int32_t num_qo_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      float sm_scale, int32_t window, void* stream) {
  sinkattn::BalancedArgs a;
  sinkattn_status st = balanced_args(q, kv, sinks, num_segments, workspace, workspace_bytes, out, lse, batch,
                                     num_qo_heads, num_kv_heads, head_dim, sm_scale, window, true, &a);
  if (st != SINKATTN_OK) return st;
  return hip_status(sinkattn::launch_decode_balanced(a, static_cast<hipStream_t>(stream)), "balanced decode launch");
}

sinkattn_status sinkattn_merge_balanced(const float* sinks, int32_t num_segments, const void* workspace,
                                        int64_t workspace_bytes, void* out, float* lse, int32_t batch,
                                        int32_t num_qo_heads, int32_t head_dim, void* stream) {
  sinkattn::BalancedArgs a;
  sinkattn_status st = balanced_args(nullptr, nullptr, sinks, num_segments, workspace, workspace_bytes, out, lse,
                                     batch, num_qo_heads, num_qo_heads, head_dim, 1.f, 0, false, &a);
  if (st != SINKATTN_OK) return st;
  return hip_status(sinkattn::launch_merge_balanced(a, static_cast<hipStream_t>(stream)), "balanced merge launch");
}

sinkattn_status sinkattn_decode_paged_balanced(const void* q, const sinkattn_kv* kv, const float* sinks,
                                               int32_t num_segments, void* workspace,
                                               int64_t workspace_bytes, void* out, float* lse,
                                               int32_t batch, int32_t num_qo_heads,
                                               int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                               int32_t window, void* stream) {
  sinkattn::BalancedArgs a;
  sinkattn_status st = balanced_args(q, kv, sinks, num_segments, workspace, workspace_bytes, out, lse, batch,
                                     num_qo_heads, num_kv_heads, head_dim, sm_scale, window, true, &a);
  if (st != SINKATTN_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(sinkattn::launch_decode_balanced(a, s), "balanced decode launch")) != SINKATTN_OK) return st;
  return hip_status(sinkattn::launch_merge_balanced(a, s), "balanced merge launch");
}

sinkattn_status sinkattn_decode_paged_multi(const void* q, const int32_t* qo_indptr,
                                            const uint8_t* custom_mask, const int32_t* mask_indptr,
                                            const sinkattn_kv* kv, const float* sinks,
                                            int32_t num_splits, void* out, float* o_part,
                                            float* lse_part, float* lse, int32_t batch,
                                            int32_t total_q, int32_t max_qo_len,
                                            int32_t num_qo_heads, int32_t num_kv_heads,
                                            int32_t head_dim, float sm_scale, int32_t window,
                                            void* stream) {
  REQUIRE(q != nullptr && qo_indptr != nullptr, SINKATTN_ERR_INVALID_ARG, "q and qo_indptr are required");
  sinkattn_status st = check_heads(batch, num_qo_heads, num_kv_heads, head_dim, sm_scale, window);
  if (st != SINKATTN_OK) return st;
  if ((st = check_kv(kv, true)) != SINKATTN_OK) return st;
  REQUIRE(total_q >= batch, SINKATTN_ERR_INVALID_ARG, "total_q (%d) must be >= batch (%d)", total_q, batch);
  const int32_t group = num_qo_heads / num_kv_heads;
  REQUIRE(max_qo_len >= 1 && max_qo_len <= SINKATTN_MAX_DECODE_ROWS, SINKATTN_ERR_INVALID_ARG,
          "max_qo_len must be in [1, %d] (got %d)", SINKATTN_MAX_DECODE_ROWS, max_qo_len);
  REQUIRE(group * max_qo_len <= 64, SINKATTN_ERR_UNSUPPORTED,
          "(Hq/Hkv) * max_qo_len = %d unsupported (at most 64)", group * max_qo_len);
  REQUIRE(num_splits >= 1 && num_splits <= SINKATTN_MAX_SPLITS, SINKATTN_ERR_INVALID_ARG,
          "num_splits must be in [1, %d] (got %d)", SINKATTN_MAX_SPLITS, num_splits);
  if (num_splits == 1) {
    REQUIRE(out != nullptr, SINKATTN_ERR_INVALID_ARG, "num_splits == 1 needs out");
  } else {
    REQUIRE(o_part != nullptr && lse_part != nullptr, SINKATTN_ERR_INVALID_ARG,
            "num_splits > 1 needs o_part and lse_part");
  }
  if (custom_mask != nullptr) {
    REQUIRE(mask_indptr != nullptr, SINKATTN_ERR_INVALID_ARG, "custom_mask needs mask_indptr");
    REQUIRE(window == 0, SINKATTN_ERR_INVALID_ARG, "a custom mask replaces the window: window must be 0");
  }
  REQUIRE((long)batch * num_kv_heads * num_splits < (1L << 31), SINKATTN_ERR_UNSUPPORTED, "launch too large");
  sinkattn::DecodeArgs d{};
  d.q = static_cast<const uint16_t*>(q);
  d.k_pool = static_cast<const uint16_t*>(kv->k);
  d.v_pool = static_cast<const uint16_t*>(kv->v);
  d.page_indptr = kv->kv_indptr;
  d.page_indices = kv->page_indices;
  d.kv_len = kv->kv_len;
  d.qo_indptr = qo_indptr;
  d.custom_mask = custom_mask;
  d.mask_indptr = custom_mask != nullptr ? mask_indptr : nullptr;
  d.sinks = sinks;
  d.out = static_cast<uint16_t*>(out);
  d.lse = lse;
  d.o_part = o_part;
  d.lse_part = lse_part;
  d.scale_log2 = sm_scale * 1.4426950408889634f;
  d.batch = batch;
  d.num_qo_heads = num_qo_heads;
  d.num_kv_heads = num_kv_heads;
  d.group = group;
  d.num_splits = num_splits;
  d.window = window;
  d.max_rows = max_qo_len;
  plan_decode_order(kv, batch, window, &d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = hip_status(sinkattn::launch_decode_verify(d, s), "verify decode launch")) != SINKATTN_OK) return st;
  if (num_splits > 1 && out != nullptr) {
    sinkattn::MergeArgs m{o_part, lse_part, static_cast<uint16_t*>(out), lse, total_q, num_qo_heads, num_splits};
    if ((st = hip_status(sinkattn::launch_merge(m, s), "merge launch")) != SINKATTN_OK) return st;
  }
  return SINKATTN_OK;
}

sinkattn_status sinkattn_append_paged_kv_rope(const void* q, const void* k_new, const void* v_new,
                                              const int32_t* append_indptr, const sinkattn_kv* kv,
                                              const float* cos_sin, int32_t max_pos,
                                              int32_t interleaved, void* q_out, int32_t batch,
                                              int32_t total_new, int32_t num_qo_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              void* stream) {
  // with no new token nothing is read or written, so the token buffers may be NULL
  REQUIRE((total_new == 0 || (k_new != nullptr && v_new != nullptr)) && append_indptr != nullptr &&
              cos_sin != nullptr,
          SINKATTN_ERR_INVALID_ARG, "k_new, v_new (unless total_new == 0), append_indptr and cos_sin are required");
  REQUIRE((q == nullptr) == (q_out == nullptr), SINKATTN_ERR_INVALID_ARG,
          "q and q_out must be given together (or both NULL)");
  sinkattn_status st = check_heads(batch, num_qo_heads, num_kv_heads, head_dim, 1.0f, 0);
  if (st != SINKATTN_OK) return st;
  if ((st = check_kv(kv, true)) != SINKATTN_OK) return st;
  REQUIRE(total_new >= 0, SINKATTN_ERR_INVALID_ARG, "total_new must be >= 0 (got %d)", total_new);
  REQUIRE(max_pos >= 1, SINKATTN_ERR_INVALID_ARG, "max_pos must be >= 1 (got %d)", max_pos);
  REQUIRE(interleaved == 0 || interleaved == 1, SINKATTN_ERR_INVALID_ARG, "interleaved must be 0 or 1");
  REQUIRE(((uintptr_t)cos_sin & 15) == 0, SINKATTN_ERR_INVALID_ARG, "cos_sin must be 16-byte aligned");
  sinkattn::AppendArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.append_indptr = append_indptr;
  a.kv_len = kv->kv_len;
  a.page_indptr = kv->kv_indptr;
  a.page_indices = kv->page_indices;
  a.cos_sin = cos_sin;
  a.q_out = static_cast<uint16_t*>(q_out);
  a.k_pool = static_cast<uint16_t*>(const_cast<void*>(kv->k));
  a.v_pool = static_cast<uint16_t*>(const_cast<void*>(kv->v));
  a.batch = batch;
  a.total_new = total_new;
  a.num_qo_heads = num_qo_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_pos = max_pos;
  a.interleaved = interleaved;
  return hip_status(sinkattn::launch_append_rope(a, static_cast<hipStream_t>(stream)), "append launch");
}

sinkattn_status sinkattn_moe_topk_softmax(const void* logits, int32_t num_tokens, int32_t num_experts,
                                          int32_t top_k, int32_t* topk_idx, void* topk_w, void* stream) {
  // with no token nothing is read or written, so the buffers may be NULL
  REQUIRE(num_tokens == 0 || (logits != nullptr && topk_idx != nullptr && topk_w != nullptr),
          SINKATTN_ERR_INVALID_ARG, "logits, topk_idx and topk_w are required");
  REQUIRE(num_tokens >= 0, SINKATTN_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
  REQUIRE(num_experts >= 1 && num_experts <= SINKATTN_MAX_EXPERTS, SINKATTN_ERR_UNSUPPORTED,
          "num_experts must be in [1, %d] (got %d)", SINKATTN_MAX_EXPERTS, num_experts);
  REQUIRE(top_k >= 1 && top_k <= SINKATTN_MAX_TOP_K && top_k <= num_experts, SINKATTN_ERR_INVALID_ARG,
          "top_k must be in [1, min(%d, num_experts)] (got %d)", SINKATTN_MAX_TOP_K, top_k);
  sinkattn::MoeArgs a{static_cast<const uint16_t*>(logits), topk_idx, static_cast<uint16_t*>(topk_w),
                      num_tokens, num_experts, top_k};
  return hip_status(sinkattn::launch_moe_topk_softmax(a, static_cast<hipStream_t>(stream)), "moe launch");
}

sinkattn_status sinkattn_merge(const float* o_part, const float* lse_part, int32_t rows,
                               int32_t num_heads, int32_t num_splits, int32_t head_dim, void* out,
                               float* lse_out, void* stream) {
  REQUIRE(o_part != nullptr && lse_part != nullptr && out != nullptr, SINKATTN_ERR_INVALID_ARG,
          "o_part, lse_part and out are required");
  REQUIRE(rows >= 1 && num_heads >= 1, SINKATTN_ERR_INVALID_ARG, "rows and num_heads must be >= 1");
  REQUIRE(num_splits >= 1 && num_splits <= SINKATTN_MAX_SPLITS, SINKATTN_ERR_INVALID_ARG,
          "num_splits must be in [1, %d] (got %d)", SINKATTN_MAX_SPLITS, num_splits);
  REQUIRE(head_dim == SINKATTN_HEAD_DIM, SINKATTN_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", head_dim);
  REQUIRE((long)rows * num_heads < (1L << 31) * 4L, SINKATTN_ERR_UNSUPPORTED, "launch too large");
  sinkattn::MergeArgs m{o_part, lse_part, static_cast<uint16_t*>(out), lse_out, rows, num_heads, num_splits};
  return hip_status(sinkattn::launch_merge(m, static_cast<hipStream_t>(stream)), "merge launch");
}

sinkattn_status sinkattn_split_bounds(const int32_t* kv_len_host, int32_t batch, int32_t page_size,
                                      int32_t num_splits, int32_t* bounds_host) {
  REQUIRE(kv_len_host != nullptr && bounds_host != nullptr, SINKATTN_ERR_INVALID_ARG,
          "kv_len_host and bounds_host are required");
  REQUIRE(batch >= 0, SINKATTN_ERR_INVALID_ARG, "batch must be >= 0");
  REQUIRE(page_size >= 1, SINKATTN_ERR_INVALID_ARG, "page_size must be >= 1");
  REQUIRE(num_splits >= 1 && num_splits <= SINKATTN_MAX_SPLITS, SINKATTN_ERR_INVALID_ARG,
          "num_splits must be in [1, %d]", SINKATTN_MAX_SPLITS);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = kv_len_host[b];
    REQUIRE(len >= 0, SINKATTN_ERR_INVALID_ARG, "kv_len[%d] < 0", b);
    const int64_t n_pages = (len + page_size - 1) / page_size;
    const int64_t ppc = (n_pages + num_splits - 1) / num_splits;
    for (int32_t c = 0; c < num_splits; ++c) {
      const int64_t p0 = c * ppc < n_pages ? c * ppc : n_pages;
      const int64_t p1 = (c + 1) * ppc < n_pages ? (c + 1) * ppc : n_pages;
      const int64_t lo = p0 * page_size < len ? p0 * page_size : len;
      const int64_t hi = p1 * page_size < len ? p1 * page_size : len;
      bounds_host[((int64_t)b * num_splits + c) * 2 + 0] = (int32_t)lo;
      bounds_host[((int64_t)b * num_splits + c) * 2 + 1] = (int32_t)hi;
    }
  }
  return SINKATTN_OK;
}

int32_t sinkattn_pick_num_splits(const int32_t* kv_len_host, int32_t batch, int32_t num_kv_heads) {
  if (kv_len_host == nullptr || batch < 1 || num_kv_heads < 1) return 1;
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) max_len = kv_len_host[b] > max_len ? kv_len_host[b] : max_len;
  const int64_t max_pages = (max_len + SINKATTN_PAGE_SIZE - 1) / SINKATTN_PAGE_SIZE;
  // aim for about eight work units per compute unit (256 CUs): the decode
  // kernel starts the longest requests first, so the dispatcher can balance
  // the rest; keep chunks at least 16 pages long, and at most 16 chunks (the
  // partials and the merge grow with the count)
  const int64_t units = (int64_t)batch * num_kv_heads;
  int64_t s = (2048 + units - 1) / units;
  const int64_t cap = max_pages / 16 > 1 ? max_pages / 16 : 1;
  if (s > cap) s = cap;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return (int32_t)s;
}

int32_t sinkattn_pick_num_splits_multi(const int32_t* kv_len_host, int32_t batch, int32_t num_qo_heads,
                                       int32_t num_kv_heads, int32_t max_qo_len, int32_t with_mask) {
  if (kv_len_host == nullptr || batch < 1 || num_kv_heads < 1 || num_qo_heads < num_kv_heads ||
      max_qo_len < 1)
    return 1;
  int64_t max_len = 0;
  for (int32_t b = 0; b < batch; ++b) max_len = kv_len_host[b] > max_len ? kv_len_host[b] : max_len;
  const int64_t max_pages = (max_len + SINKATTN_PAGE_SIZE - 1) / SINKATTN_PAGE_SIZE;
  // The several-row kernel runs two workgroups per CU (two waves per SIMD).
  // Aim for about 4/3 of the resident workgroups (twice with a mask, whose
  // pages cost more) so that one round plus a short tail covers the batch:
  // fewer, longer chunks than the one-row rule; on the verify batch (512
  // (request, KV head) units) this gives two chunks, which measured best
  // with and without masks (69.5 / 96.2 us against 74.7 / 101.6 at three).
  const int64_t per_cu = 2;
  const int64_t target = 256 * per_cu * (with_mask ? 2 : 4) / (with_mask ? 1 : 3);
  const int64_t units = (int64_t)batch * num_kv_heads;
  int64_t s = (target + units - 1) / units;
  const int64_t cap = max_pages / 16 > 1 ? max_pages / 16 : 1;
  if (s > cap) s = cap;
  if (s > 16) s = 16;
  if (s < 1) s = 1;
  return (int32_t)s;
}

const char* sinkattn_status_string(sinkattn_status status) {
  switch (status) {
    case SINKATTN_OK: return "ok";
    case SINKATTN_ERR_INVALID_ARG: return "invalid argument";
    case SINKATTN_ERR_UNSUPPORTED: return "unsupported";
    case SINKATTN_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* sinkattn_last_error(void) { return g_last_error.c_str(); }

const char* sinkattn_last_hip_error(void) { return g_last_error.c_str(); }

sinkattn_status sinkattn_validate_kv_host(const sinkattn_kv* kv, const int32_t* kv_indptr_host,
                                          const int32_t* page_indices_host,
                                          const int32_t* kv_len_host, int32_t batch) {
  REQUIRE(kv != nullptr && kv_indptr_host != nullptr, SINKATTN_ERR_INVALID_ARG,
          "kv and kv_indptr_host are required");
  REQUIRE(batch >= 0, SINKATTN_ERR_INVALID_ARG, "batch must be >= 0 (got %d)", batch);
  REQUIRE(kv->paged == 0 || kv->paged == 1, SINKATTN_ERR_INVALID_ARG, "kv->paged must be 0 or 1");
  REQUIRE(kv->num_pages >= 0, SINKATTN_ERR_INVALID_ARG, "kv->num_pages must be >= 0");
  REQUIRE(kv_indptr_host[0] >= 0, SINKATTN_ERR_INVALID_ARG, "kv_indptr[0] = %d < 0", kv_indptr_host[0]);
  for (int32_t b = 0; b < batch; ++b)
    REQUIRE(kv_indptr_host[b + 1] >= kv_indptr_host[b], SINKATTN_ERR_INVALID_ARG,
            "kv_indptr decreases at request %d (%d -> %d)", b, kv_indptr_host[b], kv_indptr_host[b + 1]);
  if (!kv->paged) {
    REQUIRE(kv_indptr_host[batch] <= kv->num_pages, SINKATTN_ERR_INVALID_ARG,
            "kv_indptr[%d] = %d exceeds the %lld rows of k and v", batch, kv_indptr_host[batch],
            (long long)kv->num_pages);
    return SINKATTN_OK;
  }
  REQUIRE(kv->page_size == SINKATTN_PAGE_SIZE, SINKATTN_ERR_UNSUPPORTED, "page_size %d unsupported (only 16)",
          kv->page_size);
  REQUIRE(kv->num_pages >= 1, SINKATTN_ERR_INVALID_ARG, "a paged pool needs num_pages >= 1");
  REQUIRE(kv_len_host != nullptr && (page_indices_host != nullptr || kv_indptr_host[batch] == kv_indptr_host[0]),
          SINKATTN_ERR_INVALID_ARG, "paged metadata needs kv_len_host and page_indices_host");
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = kv_len_host[b];
    REQUIRE(len >= 0, SINKATTN_ERR_INVALID_ARG, "kv_len[%d] = %lld < 0", b, (long long)len);
    const int64_t need = (len + SINKATTN_PAGE_SIZE - 1) / SINKATTN_PAGE_SIZE;
    const int64_t have = (int64_t)kv_indptr_host[b + 1] - kv_indptr_host[b];
    REQUIRE(need <= have, SINKATTN_ERR_INVALID_ARG,
            "request %d holds %lld keys in %lld pages but lists %lld", b, (long long)len, (long long)need,
            (long long)have);
    for (int64_t i = 0; i < need; ++i) {
      const int64_t id = page_indices_host[kv_indptr_host[b] + i];
      REQUIRE(id >= 0 && id < kv->num_pages, SINKATTN_ERR_INVALID_ARG,
              "request %d, page %lld: id %lld outside [0, %lld)", b, (long long)i, (long long)id,
              (long long)kv->num_pages);
    }
  }
  return SINKATTN_OK;
}

int32_t sinkattn_abi_version(void) { return SINKATTN_ABI_VERSION; }

}  // extern "C"
