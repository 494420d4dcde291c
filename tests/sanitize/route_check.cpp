// Host-side check built with AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Test infrastructure: links the library's host routing source (CPU-offloaded
// routing, built here without HIP) with the C oracle and runs both on small
// seeded inputs, including the degenerate ones (empty requests, anchors and
// recents covering a request, NaN / +-0 / +-inf palettes, a capacity below
// the budget, ragged column bands).  Any out-of-bounds access, leak or
// undefined operation aborts the run; a wrong result exits non-zero.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "kap.h"

// The library's error reporting lives in its HIP sources; the host routing
// code only needs these two calls.
namespace kap {
void set_error(const char*, ...) {}
kap_status fail(kap_status s, const char*, ...) { return s; }
}  // namespace kap

extern "C" {
void kor_rope(const double* x, int D, double pos, double theta, double* out);
void kor_summary(const void* K, int kv_dt, int num_pages, const int32_t* bt, int max_pages,
                 const int32_t* seq_lens, int B, int Hkv, int D, int page_size, double* out);
void kor_score(const void* q, int q_dt, const int32_t* pos, double theta, const void* summ,
               int s_dt, const int32_t* bt, int max_pages, const int32_t* seq_lens, int B, int Hq,
               int Hkv, int D, int page_size, double* scores);
void kor_proxy_query(const void* hidden, int h_dt, const void* wq, int w_dt, int B, int dm,
                     int n_out, double* out);
void kor_select(const float* scores, int B, int Hkv, int max_pages, const int32_t* seq_lens,
                int page_size, int per_head, const int32_t* anchor, const int32_t* recent,
                const int32_t* k_mid, int cap, int32_t* sel, int32_t* cnt);
int kor_budget_from_ratio(int N, int64_t s_num, int64_t s_den, int a, int r);
void kor_compact(const int32_t* sel, const int32_t* cnt, int B, int G, int cap, const int32_t* bt,
                 int max_pages, const int32_t* seq_lens, int page_size, const int32_t* pos,
                 int q_new, int32_t* cbt, int32_t* clog, int32_t* clen, int64_t* slot);
void kor_attend(const void* q, int q_dt, int q_len, const int32_t* pos0, double theta,
                double scale, const void* K, const void* V, int kv_dt, int Hkv, int D,
                int page_size, const int32_t* bt, int max_pages, const int32_t* keys,
                const int64_t* key_off, int G, int B, int Hq, double* out, double* lse);
void kor_append_kv(const void* k_new, const void* v_new, int kv_dt, const int64_t* slot, int B,
                   int q_new, int Hkv, int D, int page_size, void* K, void* V);
void kor_materialize(const void* K, const void* V, int kv_dt, int Hkv, int D, int page_size,
                     const int32_t* cbt, int B, int G, int cap, void* Kws, void* Vws,
                     int32_t* ws_table);
}

namespace {

int failures = 0;
#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      std::fprintf(stderr, __VA_ARGS__);  \
      std::fputc('\n', stderr);           \
      ++failures;                         \
    }                                     \
  } while (0)

// Seeded inputs (splitmix64); no part of the method's arithmetic.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
  float normalish() { return (float)(uniform() + uniform() + uniform() - 1.5) * 2.0f; }
  int below(int n) { return (int)(next() % (uint64_t)n); }
};

uint16_t bf16_bits(float f) {  // truncation: any bf16 value serves as an input
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

constexpr int kPs = 16;
constexpr int kF32 = 0, kBF16 = 1;

void check_select(const std::vector<float>& S, int B, int H, int P, const std::vector<int32_t>& L,
                  const std::vector<int32_t>& a, const std::vector<int32_t>& r,
                  const std::vector<int32_t>& k, int cap, const char* what) {
  for (int per_head = 0; per_head < 2; ++per_head)
    for (int threads : {1, 3}) {
      const int G = per_head ? H : 1;
      std::vector<int32_t> sel((size_t)B * G * cap), cnt((size_t)B * G);
      std::vector<int32_t> sref(sel.size()), cref(cnt.size());
      const kap_status st = kap_host_select_topk(S.data(), B, H, P, L.data(), kPs, per_head,
                                                 a.data(), r.data(), k.data(), cap, sel.data(),
                                                 cnt.data(), threads);
      CHECK(st == KAP_OK, "%s: host select status %d", what, (int)st);
      kor_select(S.data(), B, H, P, L.data(), kPs, per_head, a.data(), r.data(), k.data(), cap,
                 sref.data(), cref.data());
      CHECK(sel == sref && cnt == cref, "%s: selection differs (per_head %d, threads %d)", what,
            per_head, threads);
    }
}

}  // namespace

int main() {
  Rng rng{20260101};
  const int B = 4, Hq = 8, Hkv = 2, D = 64, P = 41;
  const std::vector<int32_t> L = {16 * 40 + 5, 16 * 20, 1, 0};
  const int pool = B * P;
  // block table: a permutation of the pool, -1 past each request's pages
  std::vector<int32_t> perm(pool);
  for (int i = 0; i < pool; ++i) perm[i] = i;
  for (int i = pool - 1; i > 0; --i) std::swap(perm[i], perm[rng.below(i + 1)]);
  std::vector<int32_t> bt((size_t)B * P, -1);
  for (int b = 0; b < B; ++b) {
    const int N = (L[b] + kPs - 1) / kPs;
    for (int p = 0; p < N; ++p) bt[(size_t)b * P + p] = perm[b * P + p];
  }
  std::vector<int32_t> pos = L;

  // ---- page scores: host routing against the oracle
  std::vector<float> q((size_t)B * Hq * D);
  for (auto& x : q) x = rng.normalish();
  std::vector<uint16_t> summ((size_t)pool * Hkv * D);
  for (auto& x : summ) x = bf16_bits(rng.normalish());
  std::vector<float> S((size_t)B * Hkv * P);
  std::vector<double> Sref(S.size());
  CHECK(kap_host_score_blocks(q.data(), pos.data(), 10000.f, summ.data(), pool, bt.data(), P,
                              L.data(), B, Hq, Hkv, D, kPs, S.data(), 3) == KAP_OK,
        "host score status");
  kor_score(q.data(), kF32, pos.data(), 10000.0, summ.data(), kBF16, bt.data(), P, L.data(), B, Hq,
            Hkv, D, kPs, Sref.data());
  double smax = 0.0;
  for (double v : Sref)
    if (std::isfinite(v)) smax = std::fmax(smax, std::fabs(v));
  for (size_t i = 0; i < S.size(); ++i) {
    if (std::isinf(Sref[i])) {
      CHECK(std::isinf(S[i]) && S[i] < 0, "score %zu: expected -inf", i);
    } else {
      CHECK(std::fabs(S[i] - Sref[i]) <= 1e-5 * smax, "score %zu: %g vs %g", i, (double)S[i],
            Sref[i]);
    }
  }

  // ---- top-K: on those scores, then on an adversarial palette with ties
  std::vector<int32_t> a = {1, 2, 0, 1}, r = {2, 3, 1, 0}, k = {9, 50, 3, 2};
  check_select(S, B, Hkv, P, L, a, r, k, 64, "scores");
  const float palette[] = {0.f, -0.f, 1.f, -1.f, 2.5f, INFINITY, -INFINITY, NAN, 1.f, 0.5f};
  std::vector<float> Sp(S.size());
  for (auto& x : Sp) x = palette[rng.below(10)];
  check_select(Sp, B, Hkv, P, L, a, r, k, 64, "palette");
  // anchors and recents covering a request, and a zero middle budget
  std::vector<int32_t> a2 = {30, 0, 1, 0}, r2 = {30, 0, 0, 5}, k2 = {4, 0, 0, 1};
  check_select(Sp, B, Hkv, P, L, a2, r2, k2, 64, "covering");
  {
    std::vector<int32_t> sel(64 * B), cnt(B);
    const kap_status st = kap_host_select_topk(S.data(), B, Hkv, P, L.data(), kPs, 0, a.data(),
                                               r.data(), k.data(), 8, sel.data(), cnt.data(), 1);
    CHECK(st == KAP_ERR_CAPACITY, "capacity below the budget: status %d", (int)st);
    CHECK(kap_host_select_topk(nullptr, 0, Hkv, P, nullptr, kPs, 0, nullptr, nullptr, nullptr, 8,
                               nullptr, nullptr, 1) == KAP_OK,
          "empty batch");
    CHECK(kap_host_select_topk(S.data(), B, Hkv, P, L.data(), kPs, 0, a.data(), r.data(), nullptr,
                               64, sel.data(), cnt.data(), 1) == KAP_ERR_INVALID_ARG,
          "null pointer");
  }

  // ---- proxy query: a ragged last band of columns and a batch past one pass
  {
    const int PB = 11, dm = 96, n = 300;
    std::vector<uint16_t> h((size_t)PB * dm), w((size_t)dm * n);
    for (auto& x : h) x = bf16_bits(rng.normalish());
    for (auto& x : w) x = bf16_bits(rng.normalish());
    std::vector<float> out((size_t)PB * n);
    std::vector<double> ref(out.size());
    CHECK(kap_host_proxy_query(h.data(), w.data(), PB, dm, n, out.data(), 4) == KAP_OK,
          "host proxy status");
    kor_proxy_query(h.data(), kBF16, w.data(), kBF16, PB, dm, n, ref.data());
    for (size_t i = 0; i < out.size(); ++i)
      CHECK(std::fabs(out[i] - ref[i]) <= 1e-4 * (1.0 + std::fabs(ref[i])), "proxy %zu: %g vs %g",
            i, (double)out[i], ref[i]);
  }

  // ---- the rest of the oracle on the same small pool (bounds and UB only)
  {
    std::vector<uint16_t> K((size_t)pool * Hkv * kPs * D), V(K.size());
    for (auto& x : K) x = bf16_bits(rng.normalish());
    for (auto& x : V) x = bf16_bits(rng.normalish());
    std::vector<double> sd((size_t)pool * Hkv * D, 0.0);
    kor_summary(K.data(), kBF16, pool, bt.data(), P, L.data(), B, Hkv, D, kPs, sd.data());
    double x[D], y[D];
    for (int d = 0; d < D; ++d) x[d] = rng.normalish();
    kor_rope(x, D, 131071.0, 1e6, y);
    CHECK(kor_budget_from_ratio(8192, 55, 1000, 1, 2) == 451, "budget from ratio");

    const int cap = 64, qn = 3;
    std::vector<int32_t> sel((size_t)B * cap), cnt(B);
    kor_select(S.data(), B, Hkv, P, L.data(), kPs, 0, a.data(), r.data(), k.data(), cap,
               sel.data(), cnt.data());
    std::vector<int32_t> cbt(sel.size()), clog(sel.size()), clen(B);
    std::vector<int64_t> slot((size_t)B * qn);
    kor_compact(sel.data(), cnt.data(), B, 1, cap, bt.data(), P, L.data(), kPs, pos.data(), qn,
                cbt.data(), clog.data(), clen.data(), slot.data());

    std::vector<uint16_t> kn((size_t)B * qn * Hkv * D), vn(kn.size());
    for (auto& v : kn) v = bf16_bits(rng.normalish());
    for (auto& v : vn) v = bf16_bits(rng.normalish());
    kor_append_kv(kn.data(), vn.data(), kBF16, slot.data(), B, qn, Hkv, D, kPs, K.data(), V.data());

    std::vector<uint16_t> Kws((size_t)B * cap * Hkv * kPs * D), Vws(Kws.size());
    std::vector<int32_t> wst(sel.size());
    kor_materialize(K.data(), V.data(), kBF16, Hkv, D, kPs, cbt.data(), B, 1, cap, Kws.data(),
                    Vws.data(), wst.data());

    // selected keys and a 2-token window over the full keys
    for (int mode = 0; mode < 2; ++mode) {
      const int ql = mode == 0 ? 1 : 2;
      std::vector<int32_t> keys;
      std::vector<int64_t> off(B + 1, 0);
      for (int b = 0; b < B; ++b) {
        if (mode == 0) {
          for (int j = 0; j < cnt[b]; ++j)
            for (int t = 0; t < kPs; ++t) {
              const int tok = sel[(size_t)b * cap + j] * kPs + t;
              if (tok < L[b]) keys.push_back(tok);
            }
        } else {
          for (int t = 0; t < L[b]; ++t) keys.push_back(t);
        }
        off[b + 1] = (int64_t)keys.size();
      }
      std::vector<float> qq((size_t)B * ql * Hq * D);
      for (auto& v : qq) v = rng.normalish();
      std::vector<double> out(qq.size()), lse((size_t)B * ql * Hq);
      kor_attend(qq.data(), kF32, ql, pos.data(), 10000.0, 0.125, K.data(), V.data(), kBF16, Hkv,
                 D, kPs, bt.data(), P, keys.empty() ? nullptr : keys.data(), off.data(), 1, B, Hq,
                 out.data(), lse.data());
      for (double v : out) CHECK(std::isfinite(v), "attend: non-finite output");
    }
  }

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("sanitized host routing and oracle: all checks passed\n");
  return 0;
}
