// Top-K page selection under the A<a>R<r>K<k> split (KRI page, A<a>R<r>K<k>
// tag section) with the lowest-index tie-break.
//
// One 1024-thread block per selection row (request, or request x KV head).
// Thread t owns the KPT consecutive pages [t*KPT, (t+1)*KPT) and keeps their
// keys in registers.  Keys are mapped to order-preserving uint32 (NaN lowest,
// -0 == +0); a 3-pass (12/10/10-bit) radix select finds the k-th largest middle key T
// and how many of the keys equal to T are still needed; an index-ordered
// block scan then admits those ties lowest index first, and a second scan
// writes the chosen pages in ascending order.  Bit-exact: integer logic only,
// apart from the pooled key, which is folded in fp32 with explicit
// round-to-nearest adds in head order and one rounded division (the KRI
// connector mean-pools over heads before the per-request top-K).
#include "kap_internal.h"

namespace kap {

constexpr int kSelectStagedPages = 11264;  // keys staged in LDS up to this table width (44 KiB)

struct SelArgs {
  const float* scores;
  int32_t Hkv, max_pages;
  const int32_t* seq_lens;
  int32_t per_head;
  const int32_t* anchor;
  const int32_t* recent;
  const int32_t* k_mid;
  int32_t cap;
  int32_t* sel;
  int32_t* cnt;
  // compact view written by the same launch (cbt == nullptr: selection only)
  const int32_t* bt;
  const int32_t* pos;
  int32_t q_new;
  int32_t* cbt;
  int32_t* clen;
  int64_t* slot;
};

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f != f) return 0u;          // NaN: below everything, all NaNs tie
  if (f == 0.f) f = 0.f;          // -0 -> +0
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix of v over the block (1024 threads, thread order); *total gets the sum.
// s_wave (33 ints) must not be reused by a later call: there is no trailing
// barrier, so each call site has its own region.
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (tid < 64) {
    const int w = tid < 16 ? s_wave[tid] : 0;
    const int inc = wave_incl_scan(w);
    if (tid < 16) s_wave[16 + tid] = inc - w;  // exclusive wave offsets
    if (tid == 15) s_wave[32] = inc;
  }
  __syncthreads();
  const int excl = s_wave[16 + wave] + x - v;
  *total = s_wave[32];
  return excl;
}

template <int KPT, bool STAGED>
__global__ __launch_bounds__(1024) void select_kernel(SelArgs a) {
  const int gr = blockIdx.x, b = blockIdx.y;
  const int G = a.per_head ? a.Hkv : 1;
  const int tid = threadIdx.x;
  __shared__ __align__(16) int s_hist[2][4096];  // radix histograms, alternating by pass
  __shared__ int s_suf[8];  // [4] keys above the chosen bin, [5] keys in it
  __shared__ int s_wave[5][33];  // one region per block scan (three passes, ties, output)
  __shared__ uint32_t s_digit;
  __shared__ int s_last;  // the row's last logical page is in its list
  if (a.cbt && tid == 0) s_last = 0;  // published by the staging barrier below
  if constexpr (!STAGED) {
    if (a.cbt) __syncthreads();  // uniform
  }
  const int nh = a.per_head ? 1 : a.Hkv;
  const float* base = a.scores + ((int64_t)b * a.Hkv + (a.per_head ? gr : 0)) * a.max_pages;
  const int32_t* btrow = a.bt ? a.bt + (int64_t)b * a.max_pages : nullptr;
  extern __shared__ float s_dyn[];  // STAGED: keys [max_pages], then (compact) the table row
  int32_t* s_bt = (int32_t*)(s_dyn + a.max_pages);
  bool bt_lds = false;  // compact view: the table row is in s_bt (block-uniform)
  if constexpr (STAGED) {
    float* s_key = s_dyn;
    if (nh == 1) {  // uniform (arguments only)
      // one score row (per-head selection, or keys pooled beforehand) and,
      // for a compact view, the request's table row for the output gather:
      // both staged whole, with straight-line loads at clamped indices that
      // wait for nothing (the row's length and split are not needed here;
      // pages outside the middle are never candidates)
      const int32_t* bsrc = btrow ? btrow : (const int32_t*)base;  // valid memory either way
      float kv[KPT];
      int btv[KPT];
#pragma unroll
      for (int u = 0; u < KPT; ++u) kv[u] = base[min(u * 1024 + tid, a.max_pages - 1)];
#pragma unroll
      for (int u = 0; u < KPT; ++u) btv[u] = bsrc[min(u * 1024 + tid, a.max_pages - 1)];
      const float sc = (float)a.Hkv;
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (u * 1024 + tid < a.max_pages)
          s_key[u * 1024 + tid] = a.per_head ? kv[u] : __fdiv_rn(kv[u], sc);
      if (a.cbt) {
#pragma unroll
        for (int u = 0; u < KPT; ++u)
          if (u * 1024 + tid < a.max_pages) s_bt[u * 1024 + tid] = btv[u];
        bt_lds = true;
      }
    }
  }
  const int L = a.seq_lens[b];
  const int N = min((max(L, 0) + kPage - 1) / kPage, a.max_pages);
  const int na = max(a.anchor[b], 0), nr = max(a.recent[b], 0), nk = a.k_mid[b];
  int32_t* out = a.sel + ((int64_t)b * G + gr) * a.cap;
  // slot mapping of the new tokens through the full table (first row of a request)
  auto write_slots = [&](const int32_t* tab) {
    if (gr != 0 || !a.slot) return;
    const long long p0 = a.pos[b];
    for (int i = tid; i < a.q_new; i += 1024) {
      const long long t = p0 + i;
      const long long p = t / kPage;
      long long sl = -1;
      if (t >= 0 && p < a.max_pages) {
        const int32_t phys = tab[p];
        if (phys >= 0) sl = (long long)phys * kPage + t % kPage;
      }
      a.slot[(int64_t)b * a.q_new + i] = sl;
    }
  };
  const bool all = (na + nr >= N);
  const int mid_lo = na, mid_hi = N - nr;
  const int take = all ? 0 : min(max(nk, 0), mid_hi - mid_lo);

  // ---- keys.  STAGED: pooled (or per-head) scores go through LDS with
  // coalesced loads (consecutive threads read consecutive pages of one head
  // row); all heads of a page are folded by one thread in head order.
  // Otherwise (very long tables) each thread reads its own pages directly.
  const int pbase = tid * KPT;
  uint32_t key[KPT];
  uint64_t cand = 0;  // bit j: page t*KPT+j is a middle candidate
  if constexpr (STAGED) {
    float* s_key = s_dyn;
    if (nh != 1 && !all) {
      // up to 8 heads x 4 pages of loads in flight per thread (more would not
      // fit the 128 registers of a 1024-thread block), folded in head order
      constexpr int SU = 4, SG = 8;
      for (int p0 = mid_lo; p0 < mid_hi; p0 += 1024 * SU) {
        float v[SU];
        for (int g0 = 0; g0 < nh; g0 += SG) {
          float w[SG][SU];
#pragma unroll
          for (int gi = 0; gi < SG; ++gi)
#pragma unroll
            for (int u = 0; u < SU; ++u) {
              const int p = p0 + u * 1024 + tid;
              w[gi][u] = (g0 + gi < nh && p < mid_hi) ? base[(int64_t)(g0 + gi) * a.max_pages + p]
                                                      : 0.f;
            }
#pragma unroll
          for (int gi = 0; gi < SG; ++gi)
#pragma unroll
            for (int u = 0; u < SU; ++u)
              if (g0 + gi < nh) v[u] = (g0 + gi == 0) ? w[gi][u] : __fadd_rn(v[u], w[gi][u]);
        }
#pragma unroll
        for (int u = 0; u < SU; ++u) {
          const int p = p0 + u * 1024 + tid;
          if (p < mid_hi) s_key[p] = a.per_head ? v[u] : __fdiv_rn(v[u], (float)a.Hkv);
        }
      }
    }
    __syncthreads();
    if (bt_lds) write_slots(s_bt);  // from the staged row: no load at the end
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = pbase + j;
      key[j] = 0u;
      if (!all && p >= mid_lo && p < mid_hi) {
        key[j] = order_key(s_key[p]);
        cand |= 1ull << j;
      }
    }
  } else {
    float kv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) kv[j] = 0.f;
    if (!all) {
      for (int g0 = 0; g0 < nh; g0 += 4) {
        float v[4][KPT];
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int j = 0; j < KPT; ++j) {
            const int p = pbase + j;
            v[gi][j] = (g0 + gi < nh && p >= mid_lo && p < mid_hi)
                           ? base[(int64_t)(g0 + gi) * a.max_pages + p] : 0.f;
          }
#pragma unroll
        for (int gi = 0; gi < 4; ++gi)
#pragma unroll
          for (int j = 0; j < KPT; ++j)
            if (g0 + gi < nh) kv[j] = (g0 + gi == 0) ? v[gi][j] : __fadd_rn(kv[j], v[gi][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = pbase + j;
      key[j] = 0u;
      if (!all && p >= mid_lo && p < mid_hi) {
        key[j] = order_key(a.per_head ? kv[j] : __fdiv_rn(kv[j], (float)a.Hkv));
        cand |= 1ull << j;
      }
    }
  }

  // ---- radix select of the take-th largest candidate key: three passes of
  // 12, 10 and 10 bits.  The first digit is wide because keys of similar
  // magnitude share their top bits: with 4096 bins the first histogram's
  // atomics spread instead of piling onto a few bins.
  uint32_t prefix = 0, pmask = 0;
  int remaining = take;
  int bin_count = 0;  // keys in the chosen bin of the last pass: after it, those equal to T
  if (take > 0) {
    // the first pass's 4096 bins and the second's 1024; each pass clears the
    // histogram the pass after it uses, before its last barrier
#pragma unroll
    for (int k = 0; k < 4; ++k) s_hist[0][k * 1024 + tid] = 0;
    s_hist[1][tid] = 0;
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int bpt = pass == 0 ? 4 : 1;  // bins per thread: 4096 or 1024 bins
      const uint32_t dmask = pass == 0 ? 0xfffu : 0x3ffu;
      int* hist = s_hist[pass & 1];
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (((cand >> j) & 1ull) && (key[j] & pmask) == prefix)
          atomicAdd(&hist[(key[j] >> shift) & dmask], 1);
      __syncthreads();
      // thread t owns bins [t * bpt, (t + 1) * bpt); the keys in bins above a
      // thread's range come from a block scan over the threads
      int hl[4];
      int local = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hl[k] = k < bpt ? hist[tid * bpt + k] : 0;
        local += hl[k];
      }
      int tot;
      const int excl = block_exclusive_scan(local, s_wave[pass], &tot);
      int above = tot - excl - local;
#pragma unroll
      for (int k = 3; k >= 0; --k) {
        if (above < remaining && above + hl[k] >= remaining) {  // one bin in the block
          s_digit = tid * bpt + k;
          s_suf[4] = above;
          s_suf[5] = hl[k];
        }
        above += hl[k];
      }
      // the third pass's histogram is the first pass's, last read above in
      // the first pass (before its final barrier)
      if (pass == 1) s_hist[0][tid] = 0;
      __syncthreads();
      const uint32_t d = s_digit;
      remaining -= s_suf[4];
      bin_count = s_suf[5];
      prefix |= d << shift;
      pmask |= dmask << shift;
      // every key of the chosen bin is taken: the digits below cannot change
      // the selection (block-uniform; the usual case after the second pass)
      if (bin_count == remaining) break;
      // the next pass rewrites s_digit / s_suf only after three more barriers
    }
  }
  // threshold on the digits fixed so far (all 32 bits unless a pass ended early)
  const uint32_t T = prefix;

  // ---- ties at T: lowest indices first.  When every key equal to T is taken
  // (the usual case: the last pass's bin holds exactly the remaining count),
  // no ranks are needed; the test is block-uniform.
  int eq_rank = 0;
  if (take > 0 && bin_count != remaining) {
    int n_eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (((cand >> j) & 1ull) && (key[j] & pmask) == T) ++n_eq;
    int tot;
    eq_rank = block_exclusive_scan(n_eq, s_wave[3], &tot);
  }

  // chosen mask, branch-free (nested branches per key cost more than the
  // arithmetic): pages outside the middle are taken whole; a middle page is
  // taken when its key is above T, or equal to T while ties remain
  const bool cands = take > 0;
  using mask_t = typename std::conditional<(KPT > 32), uint64_t, uint32_t>::type;
  mask_t chosen = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = pbase + j;
    const bool mid = !all && p >= mid_lo && p < mid_hi;
    const bool isc = cands && ((cand >> j) & 1ull);  // implies mid
    const uint32_t km = key[j] & pmask;
    const bool eq = isc && km == T;
    const bool c = p < N && (!mid || (isc && (km > T || (eq && eq_rank < remaining))));
    eq_rank += eq ? 1 : 0;
    chosen |= (mask_t)(c ? 1u : 0u) << j;
  }
  const int n_ch = KPT > 32 ? __popcll((uint64_t)chosen) : __popc((uint32_t)chosen);
  if (N > 0 && (N - 1) / KPT == tid && ((chosen >> ((N - 1) % KPT)) & 1u)) s_last = 1;
  int total;
  int pos = block_exclusive_scan(n_ch, s_wave[4], &total);  // (its barriers publish s_last)
  const int64_t row = (int64_t)b * G + gr;
  int gb[KPT];  // compact view without the staged row: one straight-line gather
  if (a.cbt && !bt_lds) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) gb[j] = btrow[min(pbase + j, a.max_pages - 1)];
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if ((chosen >> j) & 1u) {
      if (pos < a.cap) {
        out[pos] = pbase + j;
        if (a.cbt) a.cbt[row * a.cap + pos] = bt_lds ? s_bt[pbase + j] : gb[j];
      }
      ++pos;
    }
  }
  const int c = min(total, a.cap);
  for (int j = c + tid; j < a.cap; j += 1024) {
    out[j] = -1;
    if (a.cbt) a.cbt[row * a.cap + j] = -1;
  }
  if (tid == 0) a.cnt[row] = c;
  if (a.cbt) {
    // compact view: every listed page holds 16 tokens except the last logical
    // page N - 1, listed last, when it made the list (total <= capacity)
    if (tid == 0) {
      const int deficit = (s_last && total <= a.cap) ? kPage - min(kPage, L - (N - 1) * kPage) : 0;
      a.clen[row] = c * kPage - deficit;
    }
    if (!bt_lds) write_slots(btrow);
  }
}

kap_status launch_select(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                         const int32_t* seq_lens, int32_t per_head, const int32_t* anchor,
                         const int32_t* recent, const int32_t* k_mid, int32_t capacity,
                         int32_t* sel, int32_t* cnt, hipStream_t stream, const int32_t* bt,
                         const int32_t* pos, int32_t q_new, int32_t* cbt, int32_t* clen,
                         int64_t* slot) {
  SelArgs a{scores, Hkv, max_pages, seq_lens, per_head, anchor, recent, k_mid, capacity, sel, cnt,
            bt, pos, q_new, cbt, clen, slot};
  const int G = per_head ? Hkv : 1;
  dim3 grid(G, B);
  const int kpt = (max_pages + 1023) / 1024;
  const bool staged = max_pages <= kSelectStagedPages;
  const size_t lds = staged ? (size_t)max_pages * sizeof(float) * (cbt ? 2 : 1) : 0;
#define KAP_SEL(K)                                                                              \
  do {                                                                                          \
    if (staged) hipLaunchKernelGGL((select_kernel<K, true>), grid, dim3(1024), lds, stream, a); \
    else hipLaunchKernelGGL((select_kernel<K, false>), grid, dim3(1024), 0, stream, a);        \
  } while (0)
  if (kpt <= 1) KAP_SEL(1);
  else if (kpt <= 2) KAP_SEL(2);
  else if (kpt <= 4) KAP_SEL(4);
  else if (kpt <= 8) KAP_SEL(8);
  else if (kpt <= 9) KAP_SEL(9);  // a power-of-two table plus a few pages
  else if (kpt <= 12) KAP_SEL(12);
  else if (kpt <= 16) KAP_SEL(16);
  else if (kpt <= 24) KAP_SEL(24);
  else if (kpt <= 32) KAP_SEL(32);
  else if (kpt <= 48) KAP_SEL(48);
  else KAP_SEL(64);
#undef KAP_SEL
  return check_launch("select");
}

}  // namespace kap
