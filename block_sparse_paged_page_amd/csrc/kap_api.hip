// C ABI of libkap: host-side validation, workspace carving and launches.
// Every check runs before any launch; nothing here allocates or synchronizes.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <initializer_list>

#include "kap_internal.h"

namespace kap {

static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}

kap_status fail(kap_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

kap_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KAP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KAP_OK;
}

static bool dtype_ok(int32_t d) { return d == KAP_F32 || d == KAP_BF16; }

// Blocks of `kernel` the current device keeps resident at once (CUs x blocks per
// CU), cached per (device, kernel).  The only state the library keeps.
int resident_blocks(const void* kernel, int block_threads) {
  struct Entry {
    std::atomic<const void*> fn;
    std::atomic<int> dev, value;
  };
  static Entry cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  for (auto& e : cache) {
    const void* f = e.fn.load(std::memory_order_acquire);
    if (f == nullptr) break;
    if (f == kernel && e.dev.load(std::memory_order_relaxed) == dev) return e.value.load();
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block_threads, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return kTargetItems;
  }
  const int value = cus * per_cu;
  static std::atomic<int> next{0};
  const int slot = next.fetch_add(1);
  if (slot < 64) {
    cache[slot].dev.store(dev);
    cache[slot].value.store(value);
    cache[slot].fn.store(kernel, std::memory_order_release);
  }
  return value;
}

static kap_status check_heads(int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size) {
  if (Hq <= 0 || Hkv <= 0) return fail(KAP_ERR_INVALID_ARG, "Hq=%d Hkv=%d must be > 0", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(KAP_ERR_UNSUPPORTED, "Hq=%d not a multiple of Hkv=%d", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(KAP_ERR_UNSUPPORTED, "GQA group %d > 16", Hq / Hkv);
  if (D != 64 && D != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", D);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  return KAP_OK;
}

}  // namespace kap

// ------------------------------------------------------------------ allocation-free decode
// The attention workspace of kap_decode_attn_noalloc lives in this array, one
// copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): each device's address comes from hipGetSymbolAddress, taken once
// with that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[KAP_NOALLOC_SCRATCH_BYTES];

namespace kap {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (NULL on failure,
// with the error recorded).
void* scratch_address(int dev) {
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (e != hipSuccess || q == nullptr) {
    (void)hipGetLastError();
    set_error("scratch address on device %d: %s", dev, hipGetErrorString(e));
    return nullptr;
  }
  // two threads may both look it up: they find the same address
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}
}  // namespace
}  // namespace kap

using namespace kap;

extern "C" {

const char* kap_status_string(kap_status s) {
  switch (s) {
    case KAP_OK: return "ok";
    case KAP_ERR_INVALID_ARG: return "invalid argument";
    case KAP_ERR_UNSUPPORTED: return "unsupported configuration";
    case KAP_ERR_CAPACITY: return "selection budget exceeds compact capacity";
    case KAP_ERR_WORKSPACE: return "workspace too small";
    case KAP_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kap_last_error(void) { return g_err; }

const char* kap_version(void) { return "kap 0.1 gfx950"; }

// The kernels move bulk data (queries, K/V pages, summaries, weights,
// outputs, workspaces) in 16-byte vectors, some straight into LDS: those
// pointers must be 16-byte aligned (hipMalloc and torch allocations are).
static bool misaligned(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (((uintptr_t)p & 15) != 0) return true;
  return false;
}

kap_status kap_score_blocks(const void* q, int32_t q_dtype, const int32_t* positions,
                            float rope_theta, const void* summary, int32_t sum_dtype,
                            int32_t num_pages, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                            int32_t D, int32_t page_size, float* scores, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || max_pages < 0 || num_pages < 0)
    return fail(KAP_ERR_INVALID_ARG, "negative size (B=%d max_pages=%d num_pages=%d)", B,
                max_pages, num_pages);
  kap_status st = check_heads(Hq, Hkv, D, page_size);
  if (st != KAP_OK) return st;
  if (!dtype_ok(q_dtype) || !dtype_ok(sum_dtype))
    return fail(KAP_ERR_UNSUPPORTED, "dtype q=%d summary=%d", q_dtype, sum_dtype);
  if (!(rope_theta > 1.0f)) return fail(KAP_ERR_INVALID_ARG, "rope_theta %g <= 1", rope_theta);
  if (B == 0 || max_pages == 0) return KAP_OK;
  if (!q || !positions || !summary || !block_table || !seq_lens || !scores)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({q, summary})) return fail(KAP_ERR_INVALID_ARG, "q or summary not 16-byte aligned");
  return launch_score(q, (kap_dtype)q_dtype, positions, rope_theta, summary,
                      (kap_dtype)sum_dtype, block_table, max_pages, seq_lens, B, Hq, Hkv, D,
                      scores, (hipStream_t)stream);
}

kap_status kap_score_pool_blocks(const void* q, int32_t q_dtype, const int32_t* positions,
                                 float rope_theta, const void* summary, int32_t sum_dtype,
                                 int32_t num_pages, const int32_t* block_table,
                                 int32_t max_pages, const int32_t* seq_lens, int32_t B,
                                 int32_t Hq, int32_t Hkv, int32_t D, int32_t page_size,
                                 float* scores, float* pooled, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || max_pages < 0 || num_pages < 0)
    return fail(KAP_ERR_INVALID_ARG, "negative size (B=%d max_pages=%d num_pages=%d)", B,
                max_pages, num_pages);
  kap_status st = check_heads(Hq, Hkv, D, page_size);
  if (st != KAP_OK) return st;
  if (!dtype_ok(q_dtype) || !dtype_ok(sum_dtype))
    return fail(KAP_ERR_UNSUPPORTED, "dtype q=%d summary=%d", q_dtype, sum_dtype);
  if (!(rope_theta > 1.0f)) return fail(KAP_ERR_INVALID_ARG, "rope_theta %g <= 1", rope_theta);
  if (B == 0 || max_pages == 0) return KAP_OK;
  if (!q || !positions || !summary || !block_table || !seq_lens || (!pooled && !scores))
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({q, summary})) return fail(KAP_ERR_INVALID_ARG, "q or summary not 16-byte aligned");
  return launch_score_pool(q, (kap_dtype)q_dtype, positions, rope_theta, summary,
                           (kap_dtype)sum_dtype, block_table, max_pages, seq_lens, B, Hq, Hkv,
                           D, scores, pooled, (hipStream_t)stream);
}

size_t kap_proxy_workspace_bytes(int32_t B, int32_t d_model, int32_t n_out) {
  if (B <= 0 || d_model <= 0 || n_out <= 0) return 0;
  return (size_t)proxy_splits(d_model) * B * n_out * sizeof(float);
}

kap_status kap_proxy_query(const void* hidden, const void* w_q, int32_t B, int32_t d_model,
                           int32_t n_out, float* q_out, void* workspace, size_t workspace_bytes,
                           kap_stream stream) {
  g_err[0] = 0;
  if (B <= 0 || B > 16) return fail(KAP_ERR_UNSUPPORTED, "proxy batch %d (1..16)", B);
  if (d_model <= 0 || d_model % 128 != 0)
    return fail(KAP_ERR_UNSUPPORTED, "d_model %d (multiple of 128)", d_model);
  if (n_out <= 0 || n_out % 512 != 0)
    return fail(KAP_ERR_UNSUPPORTED, "n_out %d (multiple of 512)", n_out);
  if (!hidden || !w_q || !q_out) return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({hidden, w_q, q_out, workspace}))
    return fail(KAP_ERR_INVALID_ARG, "hidden, w_q, q_out or workspace not 16-byte aligned");
  const size_t need = kap_proxy_workspace_bytes(B, d_model, n_out);
  if (!workspace || workspace_bytes < need)
    return fail(KAP_ERR_WORKSPACE, "proxy workspace %zu < %zu bytes", workspace_bytes, need);
  return launch_proxy((const uint16_t*)hidden, (const uint16_t*)w_q, B, d_model, n_out, q_out,
                      (float*)workspace, proxy_splits(d_model), (hipStream_t)stream);
}

static kap_status check_packed_shape(int32_t d_model, int32_t n_out) {
  if (d_model <= 0 || d_model % 32 != 0)
    return fail(KAP_ERR_UNSUPPORTED, "d_model %d (multiple of 32)", d_model);
  if (n_out <= 0 || n_out % 16 != 0)
    return fail(KAP_ERR_UNSUPPORTED, "n_out %d (multiple of 16)", n_out);
  return KAP_OK;
}

kap_status kap_proxy_pack_weights(const void* w_q, int32_t d_model, int32_t n_out, void* w_packed,
                                  kap_stream stream) {
  g_err[0] = 0;
  kap_status st = check_packed_shape(d_model, n_out);
  if (st != KAP_OK) return st;
  if (!w_q || !w_packed) return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({w_packed})) return fail(KAP_ERR_INVALID_ARG, "w_packed not 16-byte aligned");
  if (w_q == w_packed) return fail(KAP_ERR_INVALID_ARG, "packing needs a separate output buffer");
  return launch_proxy_pack((const uint16_t*)w_q, (uint16_t*)w_packed, d_model, n_out,
                           (hipStream_t)stream);
}

kap_status kap_proxy_query_packed(const void* hidden, const void* w_packed, int32_t B,
                                  int32_t d_model, int32_t n_out, float* q_out,
                                  kap_stream stream) {
  g_err[0] = 0;
  if (B <= 0 || B > 16) return fail(KAP_ERR_UNSUPPORTED, "proxy batch %d (1..16)", B);
  kap_status st = check_packed_shape(d_model, n_out);
  if (st != KAP_OK) return st;
  if (!hidden || !w_packed || !q_out) return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({hidden, w_packed}))
    return fail(KAP_ERR_INVALID_ARG, "hidden or w_packed not 16-byte aligned");
  return launch_proxy_packed((const uint16_t*)hidden, (const uint16_t*)w_packed, B, d_model, n_out,
                             q_out, (hipStream_t)stream);
}

kap_status kap_select_topk(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                           const int32_t* seq_lens, int32_t page_size, int32_t per_head,
                           const int32_t* anchor, const int32_t* recent, const int32_t* k_mid,
                           int32_t max_budget, int32_t capacity, int32_t* sel_pages,
                           int32_t* sel_count, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || Hkv <= 0 || max_pages < 0 || capacity < 0 || max_budget < 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size (B=%d Hkv=%d max_pages=%d capacity=%d budget=%d)",
                B, Hkv, max_pages, capacity, max_budget);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (max_pages > kMaxSelectPages)
    return fail(KAP_ERR_UNSUPPORTED, "max_pages %d > %d", max_pages, kMaxSelectPages);
  if (per_head != 0 && per_head != 1) return fail(KAP_ERR_INVALID_ARG, "per_head %d", per_head);
  if (max_budget > capacity)
    return fail(KAP_ERR_CAPACITY, "budget %d pages exceeds compact capacity %d", max_budget,
                capacity);
  if (B == 0 || capacity == 0) return KAP_OK;
  if (!scores || !seq_lens || !anchor || !recent || !k_mid || !sel_pages || !sel_count)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  return launch_select(scores, B, Hkv, max_pages, seq_lens, per_head, anchor, recent, k_mid,
                       capacity, sel_pages, sel_count, (hipStream_t)stream);
}

int32_t kap_budget_from_ratio(int32_t n_pages, int64_t s_num, int64_t s_den, int32_t anchor,
                              int32_t recent) {
  if (n_pages < 0 || s_num < 0 || s_den <= 0 || anchor < 0 || recent < 0) return -1;
  int64_t budget = ((int64_t)n_pages * s_num + s_den - 1) / s_den;
  if (budget < (int64_t)anchor + recent) budget = (int64_t)anchor + recent;
  if (budget > n_pages) budget = n_pages;
  return (int32_t)budget;
}

// One layer's K and V pools in one allocation: K at byte 0, V at the K
// pool's bytes rounded up to 16 KiB plus 4 KiB.  A wave reads the K tile and
// the V tile of one (page, KV head) together; with a V offset that is a
// multiple of 16 KiB (two separate 2 MiB-aligned allocations always are),
// the two tiles share address bits 12-13 on every page.  Measured on MI355X
// at 128K, B = 4: the full-context verify took 328.7-334 us with such
// offsets (342 us at multiples of 4 MiB) against 323-326.5 us with offsets
// 4, 8 or 12 KiB past a multiple of 16 KiB; the full decode 317-322 us
// (330 us) against 317-318 us.
constexpr int64_t kKvPoolPeriod = 16384, kKvPoolShift = 4096;

kap_status kap_kv_pool_layout(int64_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t elem_bytes, int64_t* v_offset_bytes,
                              int64_t* total_bytes) {
  g_err[0] = 0;
  if (!v_offset_bytes || !total_bytes) return fail(KAP_ERR_INVALID_ARG, "null output");
  if (num_pages < 0 || num_kv_heads <= 0 || (elem_bytes != 2 && elem_bytes != 4))
    return fail(KAP_ERR_INVALID_ARG, "num_pages=%lld num_kv_heads=%d elem_bytes=%d",
                (long long)num_pages, num_kv_heads, elem_bytes);
  if (head_dim != 64 && head_dim != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  const int64_t page_bytes = (int64_t)num_kv_heads * head_dim * page_size * elem_bytes;
  if (num_pages > (INT64_MAX / 4) / page_bytes)
    return fail(KAP_ERR_INVALID_ARG, "pool of %lld pages too large", (long long)num_pages);
  const int64_t pool = num_pages * page_bytes;
  const int64_t v_off = (pool + kKvPoolPeriod - 1) / kKvPoolPeriod * kKvPoolPeriod + kKvPoolShift;
  *v_offset_bytes = v_off;
  *total_bytes = v_off + pool;
  return KAP_OK;
}

kap_status kap_choose_plan(double h, double s, double w_main_bytes, double kv_bytes, int32_t k,
                           int32_t budget_pages, int32_t capacity, int32_t* choice,
                           double* speedup) {
  g_err[0] = 0;
  // written so that NaN fails every range test
  if (!(h >= 0.0 && h <= 1.0) || !(s >= 0.0 && s <= 1.0))
    return fail(KAP_ERR_INVALID_ARG, "h=%g s=%g (both in [0, 1])", h, s);
  if (!(w_main_bytes >= 0.0) || !(kv_bytes >= 0.0) || w_main_bytes + kv_bytes == INFINITY)
    return fail(KAP_ERR_INVALID_ARG, "byte counts W_main=%g KV=%g (finite, >= 0)", w_main_bytes,
                kv_bytes);
  if (k < 1 || budget_pages < 0 || capacity < 0)
    return fail(KAP_ERR_INVALID_ARG, "k=%d budget=%d capacity=%d", k, budget_pages, capacity);
  if (!choice) return fail(KAP_ERR_INVALID_ARG, "null pointer");
  const double base = (1.0 + k * h) * (w_main_bytes + kv_bytes);
  const double plan = k * (w_main_bytes + s * kv_bytes) + (w_main_bytes + kv_bytes);
  if (speedup) *speedup = plan > 0.0 ? base / plan : 1.0;
  if (budget_pages > capacity) *choice = KAP_PLAN_FULL_CAPACITY;
  else if (!(h > s)) *choice = KAP_PLAN_FULL_MARGIN;
  else if (!((h - s) * kv_bytes > (1.0 - h) * w_main_bytes)) *choice = KAP_PLAN_FULL_BOUNDARY;
  else *choice = KAP_PLAN_SELECTED;
  return KAP_OK;
}

kap_status kap_select_compact(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                              const int32_t* seq_lens, int32_t page_size, int32_t per_head,
                              const int32_t* anchor, const int32_t* recent,
                              const int32_t* k_mid, int32_t max_budget, int32_t capacity,
                              const int32_t* block_table, const int32_t* positions,
                              int32_t q_new, int32_t* sel_count, int32_t* compact_bt,
                              int32_t* compact_logical, int32_t* compact_len,
                              int64_t* slot_mapping, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || Hkv <= 0 || max_pages < 0 || capacity < 0 || max_budget < 0 || q_new < 0)
    return fail(KAP_ERR_INVALID_ARG,
                "bad size (B=%d Hkv=%d max_pages=%d capacity=%d budget=%d q_new=%d)", B, Hkv,
                max_pages, capacity, max_budget, q_new);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (max_pages > kMaxSelectPages)
    return fail(KAP_ERR_UNSUPPORTED, "max_pages %d > %d", max_pages, kMaxSelectPages);
  if (per_head != 0 && per_head != 1) return fail(KAP_ERR_INVALID_ARG, "per_head %d", per_head);
  if (max_budget > capacity)
    return fail(KAP_ERR_CAPACITY, "budget %d pages exceeds compact capacity %d", max_budget,
                capacity);
  if (B == 0) return KAP_OK;
  if (!scores || !seq_lens || !anchor || !recent || !k_mid || !block_table || !sel_count ||
      !compact_bt || !compact_logical || !compact_len)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (q_new > 0 && (!slot_mapping || !positions))
    return fail(KAP_ERR_INVALID_ARG, "slot mapping needs positions and an output");
  return launch_select(scores, B, Hkv, max_pages, seq_lens, per_head, anchor, recent, k_mid,
                       capacity, compact_logical, sel_count, (hipStream_t)stream, block_table,
                       positions, q_new, compact_bt, compact_len,
                       q_new > 0 ? slot_mapping : nullptr);
}

kap_status kap_compact_view(const int32_t* sel_pages, const int32_t* sel_count, int32_t B,
                            int32_t G, int32_t capacity, const int32_t* block_table,
                            int32_t max_pages, const int32_t* seq_lens, int32_t page_size,
                            const int32_t* positions, int32_t q_new, int32_t* compact_bt,
                            int32_t* compact_logical, int32_t* compact_len,
                            int64_t* slot_mapping, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || G <= 0 || capacity < 0 || max_pages < 0 || q_new < 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size (B=%d G=%d capacity=%d max_pages=%d q_new=%d)", B,
                G, capacity, max_pages, q_new);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (B == 0) return KAP_OK;
  if (!sel_pages || !sel_count || !block_table || !seq_lens || !compact_bt || !compact_logical ||
      !compact_len)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (q_new > 0 && (!slot_mapping || !positions))
    return fail(KAP_ERR_INVALID_ARG, "slot mapping needs positions and an output");
  return launch_compact(sel_pages, sel_count, B, G, capacity, block_table, max_pages, seq_lens,
                        positions, q_new, compact_bt, compact_logical, compact_len,
                        q_new > 0 ? slot_mapping : nullptr, (hipStream_t)stream);
}

size_t kap_attn_workspace_bytes(int32_t B, int32_t q_len, int32_t Hq, int32_t Hkv, int32_t D) {
  if (B <= 0 || q_len <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return 0;
  return carve_attn_workspace(nullptr, B, q_len, Hq, Hkv, D).bytes;
}

static kap_status attn_common(const void* q, int32_t q_dtype, const int32_t* positions,
                              int32_t q_len, float theta, float scale, const void* k_pool,
                              const void* v_pool, int32_t kv_dtype, int32_t num_pages,
                              int32_t Hkv, int32_t D, int32_t page_size, const int32_t* table,
                              const int32_t* logical, int32_t width, int32_t G,
                              const int32_t* lens, int32_t B,
                              int32_t Hq, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, kap_stream stream) {
  if (B < 0 || width < 0 || num_pages < 0)
    return fail(KAP_ERR_INVALID_ARG, "negative size (B=%d width=%d num_pages=%d)", B, width,
                num_pages);
  kap_status st = check_heads(Hq, Hkv, D, page_size);
  if (st != KAP_OK) return st;
  if (q_len < 1 || q_len > 16) return fail(KAP_ERR_UNSUPPORTED, "q_len %d (1..16)", q_len);
  if (G != 1 && G != Hkv) return fail(KAP_ERR_INVALID_ARG, "G=%d (1 or Hkv=%d)", G, Hkv);
  if ((int64_t)B * Hkv > kMaxPlanRows)
    return fail(KAP_ERR_UNSUPPORTED, "B*Hkv=%lld > %d", (long long)B * Hkv, kMaxPlanRows);
  if (!dtype_ok(q_dtype) || !dtype_ok(kv_dtype))
    return fail(KAP_ERR_UNSUPPORTED, "dtype q=%d kv=%d", q_dtype, kv_dtype);
  if (q_dtype != kv_dtype)
    return fail(KAP_ERR_UNSUPPORTED, "q dtype %d must equal KV dtype %d", q_dtype, kv_dtype);
  if (!(theta > 1.0f)) return fail(KAP_ERR_INVALID_ARG, "rope_theta %g <= 1", theta);
  if (!(scale > 0.0f)) return fail(KAP_ERR_INVALID_ARG, "scale %g <= 0", scale);
  if (B == 0) return KAP_OK;
  if (!q || !positions || !k_pool || !v_pool || !table || !lens || !out)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({q, k_pool, v_pool, out, workspace}))
    return fail(KAP_ERR_INVALID_ARG, "q, a pool, out or workspace not 16-byte aligned");
  const size_t need = kap_attn_workspace_bytes(B, q_len, Hq, Hkv, D);
  if (!workspace || workspace_bytes < need)
    return fail(KAP_ERR_WORKSPACE, "attention workspace %zu < %zu bytes", workspace_bytes, need);
  AttnCall c{};
  c.q = q;
  c.dtype = (kap_dtype)q_dtype;
  c.positions = positions;
  c.q_len = q_len;
  c.theta = theta;
  c.scale = scale;
  c.k = k_pool;
  c.v = v_pool;
  c.Hkv = Hkv;
  c.D = D;
  c.table = table;
  c.logical = logical;
  c.width = width;
  c.G = G;
  c.lens = lens;
  c.B = B;
  c.Hq = Hq;
  c.out = out;
  c.lse = lse;
  c.ws = carve_attn_workspace(workspace, B, q_len, Hq, Hkv, D);
  c.stream = (hipStream_t)stream;
  return launch_attention(c);
}

kap_status kap_decode_attn(const void* q, int32_t q_dtype, const int32_t* positions,
                           float rope_theta, float scale, const void* k_pool, const void* v_pool,
                           int32_t kv_dtype, int32_t num_pages, int32_t Hkv, int32_t D,
                           int32_t page_size, const int32_t* block_table,
                           const int32_t* logical_table, int32_t table_width, int32_t G,
                           const int32_t* lens, int32_t B, int32_t Hq, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, kap_stream stream) {
  g_err[0] = 0;
  return attn_common(q, q_dtype, positions, 1, rope_theta, scale, k_pool, v_pool, kv_dtype,
                     num_pages, Hkv, D, page_size, block_table, logical_table, table_width, G,
                     lens, B, Hq, out, lse, workspace, workspace_bytes, stream);
}

kap_status kap_decode_attn_noalloc(const void* q, int32_t q_dtype, const int32_t* positions,
                                   float rope_theta, float scale, const void* k_pool,
                                   const void* v_pool, int32_t kv_dtype, int32_t num_pages,
                                   int32_t Hkv, int32_t D, int32_t page_size,
                                   const int32_t* block_table, const int32_t* logical_table,
                                   int32_t table_width, int32_t G, const int32_t* lens, int32_t B,
                                   int32_t Hq, void* out, float* lse, kap_stream stream) {
  g_err[0] = 0;
  // size check first, before any HIP call
  if (B > 0 && Hq > 0 && Hkv > 0 && Hq % Hkv == 0) {
    const size_t need = kap_attn_workspace_bytes(B, 1, Hq, Hkv, D);
    if (need > (size_t)KAP_NOALLOC_SCRATCH_BYTES)
      return fail(KAP_ERR_WORKSPACE,
                  "decode needs %zu bytes of scratch (B=%d Hq=%d Hkv=%d D=%d); the static "
                  "scratch holds %zu: use kap_decode_attn with a caller workspace",
                  need, B, Hq, Hkv, D, (size_t)KAP_NOALLOC_SCRATCH_BYTES);
  }
  if (B <= 0) {  // nothing to launch; validate the rest as kap_decode_attn does
    return attn_common(q, q_dtype, positions, 1, rope_theta, scale, k_pool, v_pool, kv_dtype,
                       num_pages, Hkv, D, page_size, block_table, logical_table, table_width, G,
                       lens, B, Hq, out, lse, nullptr, 0, stream);
  }
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KAP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KAP_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  void* ws = scratch_address(dev);
  if (!ws) return KAP_ERR_HIP;
  return attn_common(q, q_dtype, positions, 1, rope_theta, scale, k_pool, v_pool, kv_dtype,
                     num_pages, Hkv, D, page_size, block_table, logical_table, table_width, G,
                     lens, B, Hq, out, lse, ws, (size_t)KAP_NOALLOC_SCRATCH_BYTES, stream);
}

kap_status kap_verify_attn(const void* q, int32_t q_dtype, const int32_t* start_positions,
                           int32_t q_len, float rope_theta, float scale, const void* k_pool,
                           const void* v_pool, int32_t kv_dtype, int32_t num_pages, int32_t Hkv,
                           int32_t D, int32_t page_size, const int32_t* block_table,
                           int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t Hq,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           kap_stream stream) {
  g_err[0] = 0;
  return attn_common(q, q_dtype, start_positions, q_len, rope_theta, scale, k_pool, v_pool,
                     kv_dtype, num_pages, Hkv, D, page_size, block_table, nullptr, max_pages, 1,
                     seq_lens, B, Hq, out, lse, workspace, workspace_bytes, stream);
}

kap_status kap_build_summary(const void* k_pool, int32_t kv_dtype, int32_t num_pages,
                             int32_t Hkv, int32_t D, int32_t page_size,
                             const int32_t* block_table, int32_t max_pages,
                             const int32_t* seq_lens, int32_t B, void* summary,
                             int32_t sum_dtype, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || max_pages < 0 || num_pages < 0 || Hkv <= 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size");
  if (D != 64 && D != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", D);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (!dtype_ok(kv_dtype) || !dtype_ok(sum_dtype))
    return fail(KAP_ERR_UNSUPPORTED, "dtype kv=%d summary=%d", kv_dtype, sum_dtype);
  if (B == 0 || max_pages == 0) return KAP_OK;
  if (!k_pool || !block_table || !seq_lens || !summary)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({k_pool, summary}))
    return fail(KAP_ERR_INVALID_ARG, "k_pool or summary not 16-byte aligned");
  return launch_summary(k_pool, (kap_dtype)kv_dtype, Hkv, D, block_table, max_pages, seq_lens,
                        nullptr, 0, B, summary, (kap_dtype)sum_dtype, (hipStream_t)stream);
}

kap_status kap_update_summary(const void* k_pool, int32_t kv_dtype, int32_t num_pages,
                              int32_t Hkv, int32_t D, int32_t page_size,
                              const int32_t* block_table, int32_t max_pages,
                              const int32_t* seq_lens, const int32_t* positions, int32_t q_new,
                              int32_t B, void* summary, int32_t sum_dtype, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || max_pages < 0 || num_pages < 0 || Hkv <= 0 || q_new < 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size");
  if (D != 64 && D != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", D);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (!dtype_ok(kv_dtype) || !dtype_ok(sum_dtype))
    return fail(KAP_ERR_UNSUPPORTED, "dtype kv=%d summary=%d", kv_dtype, sum_dtype);
  if (B == 0 || max_pages == 0 || q_new == 0) return KAP_OK;
  if (!k_pool || !block_table || !seq_lens || !positions || !summary)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({k_pool, summary}))
    return fail(KAP_ERR_INVALID_ARG, "k_pool or summary not 16-byte aligned");
  return launch_summary(k_pool, (kap_dtype)kv_dtype, Hkv, D, block_table, max_pages, seq_lens,
                        positions, q_new, B, summary, (kap_dtype)sum_dtype, (hipStream_t)stream);
}

kap_status kap_materialize_view(const void* k_pool, const void* v_pool, int32_t kv_dtype,
                                int32_t num_pages, int32_t Hkv, int32_t D, int32_t page_size,
                                const int32_t* compact_bt, int32_t B, int32_t G, int32_t capacity,
                                void* k_ws, void* v_ws, int32_t ws_pages, int32_t* ws_table,
                                kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || capacity < 0 || num_pages < 0 || ws_pages < 0 || Hkv <= 0 || Hkv > 256)
    return fail(KAP_ERR_INVALID_ARG, "bad size");
  if (G != 1 && G != Hkv) return fail(KAP_ERR_INVALID_ARG, "G %d must be 1 or Hkv (%d)", G, Hkv);
  if (D != 64 && D != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", D);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (!dtype_ok(kv_dtype)) return fail(KAP_ERR_UNSUPPORTED, "dtype %d", kv_dtype);
  if ((int64_t)B * capacity > ws_pages)
    return fail(KAP_ERR_WORKSPACE, "workspace holds %d pages, B * capacity = %lld", ws_pages,
                (long long)B * capacity);
  if (B == 0 || capacity == 0) return KAP_OK;
  if (capacity > 65535 || B > 65535) return fail(KAP_ERR_UNSUPPORTED, "grid too large");
  if (!k_pool || !v_pool || !compact_bt || !k_ws || !v_ws || !ws_table)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({k_pool, v_pool, k_ws, v_ws}))
    return fail(KAP_ERR_INVALID_ARG, "a pool or workspace not 16-byte aligned");
  return launch_materialize(k_pool, v_pool, (kap_dtype)kv_dtype, Hkv, D, compact_bt, B, G,
                            capacity, k_ws, v_ws, ws_table, (hipStream_t)stream);
}

kap_status kap_append_kv(const void* k_new, const void* v_new, int32_t kv_dtype,
                         const int64_t* slot_mapping, int32_t B, int32_t q_new, int32_t Hkv,
                         int32_t D, int32_t page_size, int32_t num_pages, void* k_pool,
                         void* v_pool, kap_stream stream) {
  g_err[0] = 0;
  if (B < 0 || q_new < 0 || num_pages < 0 || Hkv <= 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size (B %d, q_new %d, Hkv %d)", B, q_new, Hkv);
  if (D != 64 && D != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", D);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (!dtype_ok(kv_dtype)) return fail(KAP_ERR_UNSUPPORTED, "dtype %d", kv_dtype);
  if ((int64_t)B * q_new > 0x7fffffffLL) return fail(KAP_ERR_UNSUPPORTED, "B * q_new too large");
  if (B == 0 || q_new == 0) return KAP_OK;
  if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({k_new, v_new, k_pool, v_pool}))
    return fail(KAP_ERR_INVALID_ARG, "new rows or a pool not 16-byte aligned");
  return launch_append(k_new, v_new, (kap_dtype)kv_dtype, slot_mapping, B, q_new, Hkv, D,
                       (int64_t)num_pages * kPage, k_pool, v_pool, (hipStream_t)stream);
}

kap_status kap_diag_stream_read(const void* buf, size_t bytes, uint32_t* sink, kap_stream stream) {
  g_err[0] = 0;
  if (!buf || !sink) return fail(KAP_ERR_INVALID_ARG, "null pointer");
  if (misaligned({buf})) return fail(KAP_ERR_INVALID_ARG, "buffer not 16-byte aligned");
  if (bytes % 16 != 0) return fail(KAP_ERR_INVALID_ARG, "bytes %zu not a multiple of 16", bytes);
  return launch_diag_read(buf, bytes, sink, (hipStream_t)stream);
}

}  // extern "C"
