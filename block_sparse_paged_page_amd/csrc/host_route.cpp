// CPU-offloaded early routing (EarlySelectKV news item, Interpretation: with
// indices available early, proxy-query construction, routing and the K-summary
// state can move to the CPU and finish before target attention; the GPU keeps
// the KV and receives only the page indices).
//
// Host code only, compiled by the host C++ compiler (no HIP): the same three
// routing steps as the GPU entry points, computed on host threads over
// host-resident inputs.  The hot loops are built for several x86-64 levels and
// picked at load time.
//   proxy query  q = hidden . W_q, fp32 sums over d_model in index order; the
//                threads split the output columns, so every column is summed
//                by one thread in one fixed order (deterministic).
//   score        u_g = sum over the group of RoPE(q_h, P) (fp64 angle reduced by
//                2 pi, fp64 rotation and group sum), then u_g . summary row in
//                fp64, rounded once to fp32.
//   top-K        the A<a>R<r>K<k> split (KRI page, tag section) with the same
//                key rules as kap_select_topk: pooled keys folded in fp32 in head
//                order and divided once by Hkv, -0 == +0, NaN below everything,
//                ties to the lower page index.  Selection is exact, so it
//                matches kap_select_topk bit for bit on the same scores.
#include <sched.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "kap.h"

namespace kap {
// the library's error reporting (kap_api.hip)
void set_error(const char* fmt, ...);
kap_status fail(kap_status s, const char* fmt, ...);

namespace {

constexpr int kPage = 16;

// Default thread count: OMP_NUM_THREADS when set (the usual per-process CPU
// share), else the CPUs this process may run on.
int default_threads() {
  if (const char* e = std::getenv("OMP_NUM_THREADS")) {
    const int n = std::atoi(e);
    if (n > 0) return n;
  }
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) == 0) return std::max(1, CPU_COUNT(&set));
  return std::max(1, (int)std::thread::hardware_concurrency());
}

int pick_threads(int requested, int work_items) {
  int t = requested > 0 ? requested : default_threads();
  t = std::max(1, std::min(t, 256));
  return std::max(1, std::min(t, work_items));
}

// Runs fn(i) for i in [0, n) on `threads` threads, contiguous ranges per thread.
template <typename F>
void parallel_for(int n, int threads, F fn) {
  if (threads <= 1 || n <= 1) {
    for (int i = 0; i < n; ++i) fn(i);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(threads);
  for (int t = 0; t < threads; ++t) {
    const int lo = (int)((int64_t)n * t / threads), hi = (int)((int64_t)n * (t + 1) / threads);
    pool.emplace_back([=, &fn] {
      for (int i = lo; i < hi; ++i) fn(i);
    });
  }
  for (auto& th : pool) th.join();
}

inline float bf16_bits_to_f32(uint16_t u) {
  const uint32_t w = (uint32_t)u << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return f;
}

// Order-preserving map of fp32 keys to uint32: NaN lowest (all NaNs equal),
// -0 == +0, otherwise the usual sign-magnitude flip.
inline uint32_t host_order_key(float f) {
  if (f != f) return 0u;
  if (f == 0.f) f = 0.f;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kProxyCols = 256;  // output columns per band (one thread's task)
constexpr int kProxyRows = 8;    // batch rows per pass over the band

// out[b][c] = sum_k h[b][k] * w[k][c] over one band of columns, k ascending.
// Each row k of the band is one contiguous run of W_q (512 bytes), so the
// walk down W_q touches one page-sized stretch per row instead of thrashing
// the TLB with narrow column strips; the 8 x 256 sums stay in L1.
__attribute__((target_clones("avx512f", "avx2", "default")))
void proxy_tile(const float* h, int nb, int dm, const uint16_t* w, size_t ldw, int nc, float* out,
                size_t ldo) {
  float acc[kProxyRows][kProxyCols] = {};
  float wf[kProxyCols];
  for (int k = 0; k < dm; ++k) {
    const uint16_t* row = w + (size_t)k * ldw;
    // rows are ldw elements apart, each in its own 4 KiB page, where the
    // hardware's stride prefetch does not follow: prefetch 8 rows ahead
    if (k + 8 < dm) {
      const char* ahead = (const char*)(row + 8 * ldw);
      for (int off = 0; off < nc * 2; off += 64) __builtin_prefetch(ahead + off);
    }
    for (int c = 0; c < nc; ++c) wf[c] = bf16_bits_to_f32(row[c]);
    for (int c = nc; c < kProxyCols; ++c) wf[c] = 0.f;
    for (int b = 0; b < nb; ++b) {
      const float hb = h[(size_t)b * dm + k];
      for (int c = 0; c < kProxyCols; ++c) acc[b][c] += hb * wf[c];
    }
  }
  for (int b = 0; b < nb; ++b)
    for (int c = 0; c < nc; ++c) out[(size_t)b * ldo + c] = acc[b][c];
}

// fp64 dot of a rotated group query with one bf16 summary row.
__attribute__((target_clones("avx512f", "avx2", "default")))
double dot_row(const double* u, const uint16_t* row, int D) {
  double s = 0.0;
  for (int d = 0; d < D; ++d) s += u[d] * (double)bf16_bits_to_f32(row[d]);
  return s;
}

}  // namespace
}  // namespace kap

using namespace kap;

extern "C" {

kap_status kap_host_proxy_query(const uint16_t* hidden, const uint16_t* w_q, int32_t B,
                                int32_t d_model, int32_t n_out, float* q_out, int32_t threads) {
  set_error("");
  if (B < 0 || d_model < 0 || n_out < 0) return fail(KAP_ERR_INVALID_ARG, "bad size");
  if (B > 64) return fail(KAP_ERR_UNSUPPORTED, "batch %d (at most 64)", B);
  if (B == 0 || n_out == 0) return KAP_OK;
  if (!hidden || !w_q || !q_out) return fail(KAP_ERR_INVALID_ARG, "null pointer");
  const int chunks = (n_out + kProxyCols - 1) / kProxyCols;
  std::vector<float> h((size_t)B * d_model);
  for (size_t i = 0; i < h.size(); ++i) h[i] = bf16_bits_to_f32(hidden[i]);
  parallel_for(chunks, pick_threads(threads, chunks), [&](int ci) {
    const int c0 = ci * kProxyCols, nc = std::min(kProxyCols, n_out - c0);
    for (int b0 = 0; b0 < B; b0 += kProxyRows)
      proxy_tile(h.data() + (size_t)b0 * d_model, std::min(kProxyRows, B - b0), d_model,
                 w_q + c0, n_out, nc, q_out + (size_t)b0 * n_out + c0, n_out);
  });
  return KAP_OK;
}

kap_status kap_host_score_blocks(const float* q, const int32_t* positions, float rope_theta,
                                 const uint16_t* summary, int32_t num_pages,
                                 const int32_t* block_table, int32_t max_pages,
                                 const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t page_size, float* scores, int32_t threads) {
  set_error("");
  if (B < 0 || max_pages < 0 || num_pages < 0 || Hq <= 0 || Hkv <= 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size");
  if (Hq % Hkv != 0) return fail(KAP_ERR_UNSUPPORTED, "Hq %d not a multiple of Hkv %d", Hq, Hkv);
  if (D != 64 && D != 128) return fail(KAP_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", D);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (!(rope_theta > 1.f)) return fail(KAP_ERR_INVALID_ARG, "rope_theta %g", rope_theta);
  if (B == 0 || max_pages == 0) return KAP_OK;
  if (!q || !positions || !summary || !block_table || !seq_lens || !scores)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  const int grp = Hq / Hkv, half = D / 2;
  const double log2_theta = std::log2((double)rope_theta);
  const double two_pi = 6.283185307179586476925286766559;
  // group-summed rotated queries u[b][g][D] in fp64
  std::vector<double> u((size_t)B * Hkv * D, 0.0);
  for (int b = 0; b < B; ++b) {
    const double P = (double)positions[b];
    for (int i = 0; i < half; ++i) {
      const double ang = P * std::exp2(-(2.0 * i / D) * log2_theta);
      const double red = ang - two_pi * std::nearbyint(ang / two_pi);
      const double c = std::cos(red), s = std::sin(red);
      for (int g = 0; g < Hkv; ++g) {
        double ux = 0.0, uy = 0.0;
        for (int hh = 0; hh < grp; ++hh) {
          const float* qh = q + ((size_t)b * Hq + (size_t)g * grp + hh) * D;
          const double x = qh[i], y = qh[i + half];
          ux += x * c - y * s;
          uy += y * c + x * s;
        }
        u[((size_t)b * Hkv + g) * D + i] = ux;
        u[((size_t)b * Hkv + g) * D + i + half] = uy;
      }
    }
  }
  // tasks: (request, run of 64 pages); a page's Hkv summary rows are one
  // contiguous block, read once for all KV heads
  constexpr int kRun = 64;
  constexpr int kAhead = 4;  // pages prefetched ahead
  const int runs = (max_pages + kRun - 1) / kRun;
  parallel_for(B * runs, pick_threads(threads, B * runs), [&](int task) {
    const int b = task / runs, p0 = (task % runs) * kRun, p1 = std::min(p0 + kRun, max_pages);
    const int L = std::max(seq_lens[b], 0);
    const int N = std::min((L + kPage - 1) / kPage, max_pages);
    for (int p = p0; p < p1; ++p) {
      if (p >= N) {
        for (int g = 0; g < Hkv; ++g) scores[((size_t)b * Hkv + g) * max_pages + p] = -INFINITY;
        continue;
      }
      // the whole summary block of the page kAhead ahead (one prefetch per
      // 64-byte line: a block is Hkv * D * 2 bytes, 2 KiB at Hkv 8, D 128)
      if (p + kAhead < N) {
        const char* nb =
            (const char*)(summary + (size_t)block_table[(size_t)b * max_pages + p + kAhead] * Hkv * D);
        for (int off = 0; off < Hkv * D * 2; off += 64) __builtin_prefetch(nb + off);
      }
      const int64_t phys = block_table[(size_t)b * max_pages + p];
      const uint16_t* blk = summary + (size_t)phys * Hkv * D;
      for (int g = 0; g < Hkv; ++g)
        scores[((size_t)b * Hkv + g) * max_pages + p] =
            (float)dot_row(u.data() + ((size_t)b * Hkv + g) * D, blk + (size_t)g * D, D);
    }
  });
  return KAP_OK;
}

kap_status kap_host_select_topk(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                                const int32_t* seq_lens, int32_t page_size, int32_t per_head,
                                const int32_t* anchor, const int32_t* recent,
                                const int32_t* k_mid, int32_t capacity, int32_t* sel_pages,
                                int32_t* sel_count, int32_t threads) {
  set_error("");
  if (B < 0 || Hkv <= 0 || max_pages < 0 || capacity < 0)
    return fail(KAP_ERR_INVALID_ARG, "bad size");
  if (per_head != 0 && per_head != 1) return fail(KAP_ERR_INVALID_ARG, "per_head %d", per_head);
  if (page_size != kPage) return fail(KAP_ERR_UNSUPPORTED, "page_size %d (16)", page_size);
  if (B == 0) return KAP_OK;
  if (!scores || !seq_lens || !anchor || !recent || !k_mid || !sel_pages || !sel_count)
    return fail(KAP_ERR_INVALID_ARG, "null pointer");
  for (int b = 0; b < B; ++b) {
    const int64_t budget = (int64_t)std::max(anchor[b], 0) + std::max(recent[b], 0) +
                           std::max(k_mid[b], 0);
    if (budget > capacity)
      return fail(KAP_ERR_CAPACITY, "request %d: budget %lld exceeds capacity %d", b,
                  (long long)budget, capacity);
  }
  const int G = per_head ? Hkv : 1;
  const int rows = B * G;
  parallel_for(rows, pick_threads(threads, rows), [&](int row) {
    const int b = row / G, gr = row % G;
    const int N = std::min((std::max(seq_lens[b], 0) + kPage - 1) / kPage, max_pages);
    const int na = std::max(anchor[b], 0), nr = std::max(recent[b], 0);
    std::vector<int32_t> chosen;
    chosen.reserve((size_t)std::min(N, capacity));
    if (na + nr >= N) {
      for (int p = 0; p < N; ++p) chosen.push_back(p);
    } else {
      const int lo = na, hi = N - nr;
      const int take = std::min(std::max(k_mid[b], 0), hi - lo);
      // (order key, page) of every middle page
      std::vector<std::pair<uint32_t, int32_t>> mid;
      mid.reserve(hi - lo);
      for (int p = lo; p < hi; ++p) {
        float key;
        if (per_head) {
          key = scores[((size_t)b * Hkv + gr) * max_pages + p];
        } else {
          float s = scores[((size_t)b * Hkv) * max_pages + p];
          for (int g = 1; g < Hkv; ++g) s = s + scores[((size_t)b * Hkv + g) * max_pages + p];
          key = s / (float)Hkv;
        }
        mid.emplace_back(host_order_key(key), p);
      }
      auto better = [](const std::pair<uint32_t, int32_t>& x, const std::pair<uint32_t, int32_t>& y) {
        return x.first != y.first ? x.first > y.first : x.second < y.second;
      };
      if (take < (int)mid.size())
        std::nth_element(mid.begin(), mid.begin() + take, mid.end(), better);
      for (int p = 0; p < lo; ++p) chosen.push_back(p);
      for (int i = 0; i < take; ++i) chosen.push_back(mid[i].second);
      for (int p = hi; p < N; ++p) chosen.push_back(p);
      std::sort(chosen.begin(), chosen.end());
    }
    const int c = std::min((int)chosen.size(), capacity);
    int32_t* out = sel_pages + (size_t)row * capacity;
    for (int j = 0; j < capacity; ++j) out[j] = j < c ? chosen[j] : -1;
    sel_count[row] = c;
  });
  return KAP_OK;
}

}  // extern "C"
