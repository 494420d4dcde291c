// Page scoring against block-mean K summaries (KRI page, KRI-Q variant:
// query-aware Q.K agreement with block-mean K, computed online).
//
// Grid (page blocks, Hkv, B); 256 threads.  Each block first forms
// u_g = sum over the GQA group of RoPE(q_h, pos) in fp64 (the rotation is
// shared by the group, so it is computed once per pair), then streams the
// 16-byte slices of its pages' summary rows: a summary row of D elements is
// read by D*eb/16 lanes, so one wave-wide load covers several pages at once
// with every byte of every touched row used.  The dot product is finished
// with xor shuffles inside the row's lanes.  HBM-bound: D*eb bytes per
// (page, KV head) plus the 4-byte table entry and the 4-byte score written.
#include "kap_internal.h"

namespace kap {

struct ScoreArgs {
  const void* q;
  const int32_t* pos;
  double log2_theta;
  const void* summ;
  const int32_t* bt;
  int32_t max_pages;
  const int32_t* seq_lens;
  int32_t Hq, Hkv, grp;
  float* scores;
};

constexpr int kScorePagesPerBlock = 256;

template <typename T>
__device__ __forceinline__ double widen_any(const void* p, int64_t i) {
  return (double)load_as_f32<T>((const T*)p, i);
}

template <int D, typename ST, typename QT>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int EPL = 16 / (int)sizeof(ST);  // elements per 16-byte load
  constexpr int LPR = D / EPL;               // lanes per summary row
  constexpr int RPL = 64 / LPR;              // rows per wave-wide load
  const int part = lane % LPR, sub = lane / LPR;
  const int N = (a.seq_lens[b] + kPage - 1) / kPage;
  const int blk0 = blockIdx.x * kScorePagesPerBlock;
  constexpr int per_wave = kScorePagesPerBlock / 4;
  constexpr int U = per_wave / RPL;  // pages per lane group, all loads in flight at once
  const int w0 = blk0 + wave * per_wave;
  const int w1 = min(w0 + per_wave, a.max_pages);
  const int32_t* btrow = a.bt + (int64_t)b * a.max_pages;
  float* out = a.scores + ((int64_t)b * a.Hkv + g) * a.max_pages;
  const ST* summ = (const ST*)a.summ;

  // The group's query heads are fetched first, then the wave's page-table
  // entries (lane j: page w0 + j) and every summary row the lane needs; the
  // group query is rotated and summed while the summary rows are in flight.
  __shared__ float su[D];
  __shared__ float sq[16 * D];  // the group's query heads (grp <= 16)
  constexpr int QPT = 16 * D / 256;
  float qv[QPT];
  {
    const int64_t q0 = ((int64_t)b * a.Hq + g * a.grp) * D;  // group heads are contiguous
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int e = k * 256 + tid;
      qv[k] = e < a.grp * D ? (float)widen_any<QT>(a.q, q0 + e) : 0.f;
    }
  }
  const int tr = (w0 + lane < min(w1, N)) ? btrow[w0 + lane] : 0;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = u * RPL + sub;
    const int64_t phys = __shfl(tr, j);
    v[u] = make_uint4(0, 0, 0, 0);
    if (w0 + j < N && w0 + j < w1)
      v[u] = *(const uint4*)(summ + (phys * a.Hkv + g) * D + part * EPL);
  }
#pragma unroll
  for (int k = 0; k < QPT; ++k) sq[k * 256 + tid] = qv[k];
  __syncthreads();
  constexpr int half = D / 2;
  for (int pair = tid; pair < half; pair += 256) {
    double s, c;
    rope_sincos((double)a.pos[b], pair, D, a.log2_theta, &s, &c);
    double ux = 0.0, uy = 0.0;
    for (int hh = 0; hh < a.grp; ++hh) {
      const double x = sq[hh * D + pair];
      const double y = sq[hh * D + pair + half];
      ux += x * c - y * s;
      uy += y * c + x * s;
    }
    su[pair] = (float)ux;
    su[pair + half] = (float)uy;
  }
  __syncthreads();
  float ur[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) ur[e] = su[part * EPL + e];

#pragma unroll
  for (int u = 0; u < U; ++u) {
    float dot = 0.f;
    if constexpr (sizeof(ST) == 2) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dot += ur[2 * e] * __uint_as_float(w[e] << 16);
        dot += ur[2 * e + 1] * __uint_as_float(w[e] & 0xffff0000u);
      }
    } else {
      dot += ur[0] * __uint_as_float(v[u].x);
      dot += ur[1] * __uint_as_float(v[u].y);
      dot += ur[2] * __uint_as_float(v[u].z);
      dot += ur[3] * __uint_as_float(v[u].w);
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) dot += __shfl_xor(dot, m);
    const int p = w0 + u * RPL + sub;
    if (part == 0 && p < w1) out[p] = (p < N) ? dot : -INFINITY;
  }
}

kap_status launch_score(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                        const void* summ, kap_dtype s_dt, const int32_t* bt, int32_t max_pages,
                        const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                        float* scores, hipStream_t stream) {
  ScoreArgs a{q, pos, log2((double)theta), summ, bt, max_pages, seq_lens, Hq, Hkv, Hq / Hkv,
              scores};
  dim3 grid((max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, Hkv, B);
#define KAP_SCORE_LAUNCH(DD, ST, QT) \
  hipLaunchKernelGGL((score_kernel<DD, ST, QT>), grid, dim3(256), 0, stream, a)
  const bool sb = s_dt == KAP_BF16, qb = q_dt == KAP_BF16;
  if (D == 128) {
    if (sb && qb) KAP_SCORE_LAUNCH(128, uint16_t, uint16_t);
    else if (sb) KAP_SCORE_LAUNCH(128, uint16_t, float);
    else if (qb) KAP_SCORE_LAUNCH(128, float, uint16_t);
    else KAP_SCORE_LAUNCH(128, float, float);
  } else {
    if (sb && qb) KAP_SCORE_LAUNCH(64, uint16_t, uint16_t);
    else if (sb) KAP_SCORE_LAUNCH(64, uint16_t, float);
    else if (qb) KAP_SCORE_LAUNCH(64, float, uint16_t);
    else KAP_SCORE_LAUNCH(64, float, float);
  }
#undef KAP_SCORE_LAUNCH
  return check_launch("score");
}

}  // namespace kap
