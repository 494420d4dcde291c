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
  float* pooled;
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
    // unconditional loads at clamped indices: a load under a branch makes
    // the compiler wait for it (and every older load) before going on
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int e = k * 256 + tid;
      const float x = (float)widen_any<QT>(a.q, q0 + min(e, a.grp * D - 1));
      qv[k] = e < a.grp * D ? x : 0.f;
    }
  }
  const int tr0 = btrow[min(w0 + lane, a.max_pages - 1)];
  const int tr = (w0 + lane < min(w1, N)) ? tr0 : 0;
  // every lane's page ids first (one LDS round trip), then all row loads
  int phys[U];
#pragma unroll
  for (int u = 0; u < U; ++u) phys[u] = __shfl(tr, u * RPL + sub);
  uint4 v[U];  // summary rows are read once per call: streaming loads
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int j = u * RPL + sub;
    v[u] = make_uint4(0, 0, 0, 0);
    if (w0 + j < N && w0 + j < w1)
      v[u] = ld_stream16(summ + ((int64_t)phys[u] * a.Hkv + g) * D + part * EPL);
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

// All KV heads of a run of pages in one block, with the head-pooled key.
// Grid (B, runs of 32 pages); one wave per KV head (Hkv <= 16).  Each wave
// reads its head's 32 summary rows exactly as score_kernel does (same access
// pattern and arithmetic, so the per-head scores are the same), and the waves
// of a block read the same 32 pages, so each page's contiguous run of head
// rows is fetched together.  The run's scores are then folded over the heads
// in head order, in fp32 with round-to-nearest adds and one rounded division:
// the same mean the top-K forms for pooled selection, so the top-K then reads
// one key row per request instead of Hkv.
// Order of a wave's work: the table entries and the group's query heads are
// requested at once (clamped indices, no wait for the request's length), the
// rotation angles are computed from the position while they are in flight,
// the summary rows are requested as soon as the table entries land, and the
// group query is rotated and summed in the wave's own LDS region while the
// rows are in flight.  Only the fold over heads needs the whole block.
// Pages per block: at most 32 (eight 16-byte row loads in flight per lane at
// D = 128 in bf16).  Runs of 64 pages gave 320 blocks for 8 requests of 40K
// tokens, so a quarter of the CUs held two blocks and set the end: 32-page
// runs took that scoring call from 12.4-13.0 to 10.1-10.4 us, and the 128K
// pooled scoring from 15.3-15.7 to 13.7-15.4 us (runs of 16, 24 and 48
// pages: no better at 40K, slower at 128K).
template <int D, typename ST>
constexpr int pool_pages_per_block() {
  return 16 * (64 / (D / (16 / (int)sizeof(ST)))) < 32 ? 16 * (64 / (D / (16 / (int)sizeof(ST))))
                                                        : 32;
}
constexpr int kPoolMaxHeads = 16;
constexpr size_t kPoolMaxQueryLds = 64 * 1024;

// Bytes of LDS a wave stages its group's query heads in: whole 1 KiB blocks
// (one 16-byte load per lane each), so a block's last load may run past the
// group's rows into padding.
template <typename QT>
__host__ __device__ constexpr int pool_query_region(int grp, int D) {
  return (grp * D * (int)sizeof(QT) + 1023) / 1024 * 1024;
}

// Dynamic LDS of score_pool_kernel: one query region per wave.
inline size_t pool_query_lds(kap_dtype q_dt, int Hq, int Hkv, int D) {
  const int grp = Hq / Hkv;
  return (size_t)Hkv * (q_dt == KAP_BF16 ? pool_query_region<uint16_t>(grp, D)
                                         : pool_query_region<float>(grp, D));
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

template <int D, typename ST, typename QT>
__global__ __launch_bounds__(1024) void score_pool_kernel(ScoreArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, g = tid >> 6;
  const int nt = blockDim.x;  // 64 * Hkv
  constexpr int EPL = 16 / (int)sizeof(ST);
  constexpr int LPR = D / EPL;
  constexpr int RPL = 64 / LPR;
  constexpr int PPB = pool_pages_per_block<D, ST>();  // pages per block (<= 64)
  constexpr int U = PPB / RPL;
  constexpr int half = D / 2;
  constexpr int QC = D * (int)sizeof(QT) / 64;  // 1 KiB query blocks per wave at most (grp <= 16)
  const int part = lane % LPR, sub = lane / LPR;
  const int w0 = blockIdx.y * PPB;
  const int w1 = min(w0 + PPB, a.max_pages);
  const ST* summ = (const ST*)a.summ;
  extern __shared__ __align__(16) unsigned char smem[];
  // wave g's region: its group's query heads, then padding (written and read
  // by that wave only, so staging needs no block barrier)
  const int qreg = pool_query_region<QT>(a.grp, D);
  unsigned char* sqg = smem + (size_t)g * qreg;
  __shared__ float su[kPoolMaxHeads][D];
  __shared__ float sc[kPoolMaxHeads][PPB];
  __shared__ int sbt[kPoolMaxHeads][64];

  // The group's query heads and the run's table entries go straight to LDS
  // (global_load_lds: no registers, and the compiler keeps them where they
  // stand), all issued before the request's length is known; the length and
  // position come by scalar loads beside them.  Clamped sources: lanes past
  // the group's rows fill the region's padding.
  const int L = a.seq_lens[b], P = a.pos[b];  // scalar loads, ahead of the LDS writes
  const int nchunk = a.grp * D * (int)sizeof(QT) / 16;
  const uint4* qsrc = (const uint4*)((const QT*)a.q + ((int64_t)b * a.Hq + (int64_t)g * a.grp) * D);
#pragma unroll
  for (int k = 0; k < QC; ++k)
    if (k * 1024 < qreg)  // uniform
      __builtin_amdgcn_global_load_lds((gptr_t)(qsrc + min(k * 64 + lane, nchunk - 1)),
                                       (lptr_t)(sqg + k * 1024), 16, 0, 0);
  __builtin_amdgcn_global_load_lds(
      (gptr_t)(a.bt + (int64_t)b * a.max_pages + min(w0 + lane, a.max_pages - 1)),
      (lptr_t)&sbt[g][0], 4, 0, 0);
  const int N = (L + kPage - 1) / kPage;
  double sn = 0.0, cs = 1.0;  // lane = rotation pair; the angle needs only the position
  if (lane < half) rope_sincos((double)P, lane, D, a.log2_theta, &sn, &cs);
  const int nv = max(0, min(w1, N) - w0);  // pages of the run that hold keys

  if (nv > 0) {  // uniform over the block
    // every load above has landed (loads complete in order; the table
    // entries were issued last)
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    // rows past the run's keys re-read its first page (masked below), so
    // every lane issues the same straight-line loads
    int phys[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = u * RPL + sub;
      phys[u] = sbt[g][j < nv ? j : 0];
    }
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = ld_stream16(summ + ((int64_t)phys[u] * a.Hkv + g) * D + part * EPL);
    // u_g = sum over the group of RoPE(q_h, pos), while the rows are in flight
    const QT* qg = (const QT*)sqg;
    if (lane < half) {
      double ux = 0.0, uy = 0.0;
      for (int hh = 0; hh < a.grp; ++hh) {
        const double x = load_as_f32<QT>(qg, hh * D + lane);
        const double y = load_as_f32<QT>(qg, hh * D + lane + half);
        ux += x * cs - y * sn;
        uy += y * cs + x * sn;
      }
      su[g][lane] = (float)ux;
      su[g][lane + half] = (float)uy;
    }
    // LDS operations of one wave complete in order: the reads below see
    // every lane's writes without a barrier (this keeps the compiler's order)
    __builtin_amdgcn_wave_barrier();
    float ur[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) ur[e] = su[g][part * EPL + e];
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
      const int j = u * RPL + sub;
      if (part == 0) sc[g][j] = (j < nv) ? dot : -INFINITY;
    }
    lds_barrier();
  }
  // per-head scores along the run (coalesced) and the pooled key
  const int np = w1 - w0;
  if (a.scores) {
    for (int e = tid; e < a.Hkv * PPB; e += nt) {
      const int gg = e / PPB, j = e % PPB;
      if (j < np)
        a.scores[((int64_t)b * a.Hkv + gg) * a.max_pages + w0 + j] = j < nv ? sc[gg][j] : -INFINITY;
    }
  }
  if (a.pooled && tid < np) {  // np <= 64 <= 64 * Hkv threads
    float k = -INFINITY;
    if (tid < nv) {
      k = sc[0][tid];
      for (int gg = 1; gg < a.Hkv; ++gg) k = __fadd_rn(k, sc[gg][tid]);
      k = __fdiv_rn(k, (float)a.Hkv);
    }
    a.pooled[(int64_t)b * a.max_pages + w0 + tid] = k;
  }
}

kap_status launch_score(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                        const void* summ, kap_dtype s_dt, const int32_t* bt, int32_t max_pages,
                        const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                        float* scores, hipStream_t stream) {
  // Up to 16 KV heads the all-heads kernel computes the same per-head scores
  // (same loads and arithmetic per head) and reads each page's head rows
  // together, which measured faster; this kernel serves the other shapes.
  if (Hkv <= kPoolMaxHeads && pool_query_lds(q_dt, Hq, Hkv, D) <= kPoolMaxQueryLds)
    return launch_score_pool(q, q_dt, pos, theta, summ, s_dt, bt, max_pages, seq_lens, B, Hq, Hkv,
                             D, scores, nullptr, stream);
  ScoreArgs a{q, pos, log2((double)theta), summ, bt, max_pages, seq_lens, Hq, Hkv, Hq / Hkv,
              scores, nullptr};
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

kap_status launch_score_pool(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                             const void* summ, kap_dtype s_dt, const int32_t* bt,
                             int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t D, float* scores, float* pooled,
                             hipStream_t stream) {
  if (Hkv > kPoolMaxHeads)
    return fail(KAP_ERR_UNSUPPORTED, "pooled scoring with Hkv=%d > %d", Hkv, kPoolMaxHeads);
  ScoreArgs a{q, pos, log2((double)theta), summ, bt, max_pages, seq_lens, Hq, Hkv, Hq / Hkv,
              scores, pooled};
  const size_t lds = pool_query_lds(q_dt, Hq, Hkv, D);
  if (lds > kPoolMaxQueryLds)
    return fail(KAP_ERR_UNSUPPORTED, "pooled scoring stages %zu query bytes (> %zu)", lds,
                kPoolMaxQueryLds);
  const int ppb = s_dt == KAP_BF16 ? (D == 128 ? pool_pages_per_block<128, uint16_t>()
                                                : pool_pages_per_block<64, uint16_t>())
                                   : (D == 128 ? pool_pages_per_block<128, float>()
                                               : pool_pages_per_block<64, float>());
  dim3 grid(B, (max_pages + ppb - 1) / ppb);
#define KAP_POOL_LAUNCH(DD, ST, QT) \
  hipLaunchKernelGGL((score_pool_kernel<DD, ST, QT>), grid, dim3(64 * Hkv), lds, stream, a)
  const bool sb = s_dt == KAP_BF16, qb = q_dt == KAP_BF16;
  if (D == 128) {
    if (sb && qb) KAP_POOL_LAUNCH(128, uint16_t, uint16_t);
    else if (sb) KAP_POOL_LAUNCH(128, uint16_t, float);
    else if (qb) KAP_POOL_LAUNCH(128, float, uint16_t);
    else KAP_POOL_LAUNCH(128, float, float);
  } else {
    if (sb && qb) KAP_POOL_LAUNCH(64, uint16_t, uint16_t);
    else if (sb) KAP_POOL_LAUNCH(64, uint16_t, float);
    else if (qb) KAP_POOL_LAUNCH(64, float, uint16_t);
    else KAP_POOL_LAUNCH(64, float, float);
  }
#undef KAP_POOL_LAUNCH
  return check_launch("score_pool");
}

}  // namespace kap
