// Compact view over a page selection (KAP paper, selected-KV view): a compact
// table lists the physical page of every chosen logical page, in ascending
// logical order, beside the logical page itself (positions stay logical), and
// the slot mapping gives each new token its physical page and offset.
//
// One 256-thread block per selection row: gather the physical page of every
// selected logical page, count the row's valid tokens (block reduction) and,
// for the first row of each request, emit the slot mapping of the new tokens
// through the full table.  Also: block-mean K summaries (the K-summary cache
// that the scorer reads), one block per (logical page, request).
#include "kap_internal.h"

namespace kap {

struct CompactArgs {
  const int32_t* sel;
  const int32_t* cnt;
  int32_t G, cap;
  const int32_t* bt;
  int32_t max_pages;
  const int32_t* seq_lens;
  const int32_t* pos;
  int32_t q_new;
  int32_t* cbt;
  int32_t* clog;
  int32_t* clen;
  int64_t* slot;
};

__global__ __launch_bounds__(256) void compact_kernel(CompactArgs a) {
  const int gr = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)b * a.G + gr;
  const int L = a.seq_lens[b];
  const int c = min(max(a.cnt[row], 0), a.cap);
  const int32_t* srow = a.sel + row * a.cap;
  const int32_t* btrow = a.bt + (int64_t)b * a.max_pages;
  long long tokens = 0;
  for (int j = tid; j < a.cap; j += 256) {
    int32_t phys = -1, lg = -1;
    if (j < c) {
      const int p = srow[j];
      if (p >= 0 && p < a.max_pages) {
        phys = btrow[p];
        lg = p;
        tokens += max(0, min(kPage, L - p * kPage));
      }
    }
    a.cbt[row * a.cap + j] = phys;
    a.clog[row * a.cap + j] = lg;
  }
  __shared__ long long s_sum[4];
  for (int o = 32; o > 0; o >>= 1) tokens += __shfl_xor(tokens, o);
  if ((tid & 63) == 0) s_sum[tid >> 6] = tokens;
  __syncthreads();
  if (tid == 0) a.clen[row] = (int32_t)(s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3]);
  if (gr == 0 && a.slot) {
    for (int i = tid; i < a.q_new; i += 256) {
      const long long t = (long long)a.pos[b] + i;
      const long long p = t / kPage;
      long long s = -1;
      if (t >= 0 && p < a.max_pages) {
        const int32_t phys = btrow[p];
        if (phys >= 0) s = (long long)phys * kPage + t % kPage;
      }
      a.slot[(int64_t)b * a.q_new + i] = s;
    }
  }
}

kap_status launch_compact(const int32_t* sel, const int32_t* cnt, int32_t B, int32_t G,
                          int32_t cap, const int32_t* bt, int32_t max_pages,
                          const int32_t* seq_lens, const int32_t* pos, int32_t q_new,
                          int32_t* cbt, int32_t* clog, int32_t* clen, int64_t* slot,
                          hipStream_t stream) {
  CompactArgs a{sel, cnt, G, cap, bt, max_pages, seq_lens, pos, q_new, cbt, clog, clen, slot};
  hipLaunchKernelGGL(compact_kernel, dim3(G, B), dim3(256), 0, stream, a);
  return check_launch("compact");
}

// ------------------------------------------------------------------ K summaries
struct SummaryArgs {
  const void* k;
  int32_t Hkv, D;
  const int32_t* bt;
  int32_t max_pages;
  const int32_t* seq_lens;
  const int32_t* first_pos;  // nullptr: all pages; else the pages of a token window
  int32_t q_new;
  void* summ;
};

template <typename KT, typename ST>
__global__ __launch_bounds__(256) void summary_kernel(SummaryArgs a) {
  const int b = blockIdx.y;
  int p = blockIdx.x;
  if (a.first_pos) {  // window [P, P + q_new): pages P/16 .. (P + q_new - 1)/16
    const int P = a.first_pos[b];
    const int t0 = max(P, 0), t1 = P + a.q_new - 1;
    if (t1 < t0) return;
    p += t0 / kPage;
    if (p > t1 / kPage) return;
  }
  const int L = a.seq_lens[b];
  const int N = min((max(L, 0) + kPage - 1) / kPage, a.max_pages);
  if (p >= N) return;
  const int nvalid = min(kPage, L - p * kPage);
  const int64_t phys = a.bt[(int64_t)b * a.max_pages + p];
  const KT* kp = (const KT*)a.k + phys * a.Hkv * kPage * a.D;
  for (int e = threadIdx.x; e < a.Hkv * a.D; e += 256) {
    const int g = e / a.D, d = e % a.D;
    float s = 0.f;
    for (int t = 0; t < nvalid; ++t) s += load_as_f32<KT>(kp, ((int64_t)g * kPage + t) * a.D + d);
    const float mean = __fdiv_rn(s, (float)nvalid);
    const int64_t o = (phys * a.Hkv + g) * a.D + d;
    if constexpr (sizeof(ST) == 2) ((uint16_t*)a.summ)[o] = f32_to_bf16(mean);
    else ((float*)a.summ)[o] = mean;
  }
}

kap_status launch_summary(const void* k, kap_dtype kv_dt, int32_t Hkv, int32_t D,
                          const int32_t* bt, int32_t max_pages, const int32_t* seq_lens,
                          const int32_t* first_pos, int32_t q_new, int32_t B, void* summ,
                          kap_dtype s_dt, hipStream_t stream) {
  SummaryArgs a{k, Hkv, D, bt, max_pages, seq_lens, first_pos, q_new, summ};
  // a window of q_new tokens spans at most (q_new - 1) / 16 + 2 pages
  const int span = first_pos ? min(max_pages, (q_new - 1) / kPage + 2) : max_pages;
  dim3 grid(span, B);
  if (kv_dt == KAP_BF16 && s_dt == KAP_BF16)
    hipLaunchKernelGGL((summary_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, stream, a);
  else if (kv_dt == KAP_BF16)
    hipLaunchKernelGGL((summary_kernel<uint16_t, float>), grid, dim3(256), 0, stream, a);
  else if (s_dt == KAP_BF16)
    hipLaunchKernelGGL((summary_kernel<float, uint16_t>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((summary_kernel<float, float>), grid, dim3(256), 0, stream, a);
  return check_launch("summary");
}

}  // namespace kap
