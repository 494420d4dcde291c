// Proxy query for early routing (EarlySelectKV news item, Interpretation: the
// side flow projects a preceding hidden state through the query projection to
// obtain the routing query).  q_out = hidden @ W_q, bf16 inputs, fp32 sums.
//
// HBM-bound GEMV (B <= 16 rows share each W_q byte) in two launches: each row
// split of kProxyRows rows of W_q forms its partial sums (on the matrix cores,
// below), the kProxyGroup splits of a block add theirs in split order through
// LDS and write one partial per group, and a second kernel adds the groups in
// group order (deterministic).
#include "kap_internal.h"

namespace kap {

constexpr int kProxyRows = 128;  // W_q rows per split

// Partial sums on the matrix cores.  hidden [B][dm] @ W_q [dm][n]
// is a dense contraction with M = B <= 16 (padded to 16), so it runs as
// v_mfma_f32_16x16x32_bf16 with A = the hidden rows and B = W_q.  One wave
// owns 128 output columns x kProxyRows rows of W_q (one row split).  Lane
// (i, j) = (lane % 16, lane / 16) loads, for each 32-row k-step, rows
// 8j .. 8j+7 of the step at columns 8i .. 8i+7 (eight 16-byte loads; each
// load instruction covers four 256-byte row segments), so it holds an 8 x 8
// tile of W_q.  The MFMA wants, per lane, 8 consecutive k of one column; MFMA
// t (t = 0..7) takes column 8i + t from lane i, so each lane only transposes
// its own tile (byte permutes, no exchange between lanes), and the eight
// MFMAs of a step cover the 128 columns with column 8i + t in lane i of
// instance t.  Products of bf16 are exact in fp32 and the matrix cores add in
// fp32 (a different order than the lane loop: results agree to fp32 rounding).
// All four k-steps' loads go out before the first MFMA (W_q is read once per
// call: streaming loads), with the hidden slices first.  The B x 8 outputs a
// lane holds (rows 4j .. 4j+3 of each MFMA) are added over the block's
// splits and go to the group's partial sums.  Four waves per block (one
// group) keep 1024 waves on all 256 CUs for a 4096 x 4096 W_q, and write a
// quarter of the partial sums that one wave per split would (B = 8: 4 MiB ->
// 1 MiB, which the second kernel then reads): 11.1-11.3 -> 10.7-10.9 us per
// call.
constexpr int kProxyMfmaCols = 128;
constexpr int kProxyGroup = 4;  // row splits per block, added in LDS
__global__ __launch_bounds__(64 * kProxyGroup) void proxy_mfma_kernel(const uint16_t* hidden,
                                                        const uint16_t* wq, int B, int dm,
                                                        int n_out, float* partial) {
  const int n0 = blockIdx.x * kProxyMfmaCols;
  const int wv = threadIdx.x >> 6;
  const int splits = dm / kProxyRows;
  const int split = min(blockIdx.y * kProxyGroup + wv, splits - 1);
  const bool live = blockIdx.y * kProxyGroup + wv < splits;
  const int c0 = split * kProxyRows;
  const int lane = threadIdx.x & 63, i = lane & 15, j = lane >> 4;
  constexpr int KSTEPS = kProxyRows / 32;
  // hidden rows (A operand): lane (i, j) holds hidden[i][k + 8j .. + 7]; rows
  // past B load row B - 1 and are masked to zero (straight-line loads)
  uint4 hf[KSTEPS];
  const uint16_t* hrow = hidden + (int64_t)min(i, B - 1) * dm + c0 + 8 * j;
  const uint32_t keep = i < B ? 0xffffffffu : 0u;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const uint4 x = *(const uint4*)(hrow + 32 * s);
    hf[s] = make_uint4(x.x & keep, x.y & keep, x.z & keep, x.w & keep);
  }
  // W_q tiles: w[s][r] = row c0 + 32 s + 8 j + r, columns n0 + 8 i .. + 7
  uint4 w[KSTEPS][8];
  const uint16_t* wbase = wq + (int64_t)(c0 + 8 * j) * n_out + n0 + 8 * i;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int r = 0; r < 8; ++r) w[s][r] = ld_stream16(wbase + (int64_t)(32 * s + r) * n_out);
  floatx4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, hf[s]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      // column t of the tile, 8 rows: dword m = (row 2m, row 2m + 1)
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
      uint32_t d[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = (&w[s][2 * m].x)[t >> 1], hi = (&w[s][2 * m + 1].x)[t >> 1];
        d[m] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      const bf16x8 bv = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bv, acc[t], 0, 0, 0);
    }
  }
  // the group's splits added in split order through LDS (a wave past the
  // last split read a copy of it and adds zeros)
  __shared__ floatx4 red[kProxyGroup][8][64];
#pragma unroll
  for (int t = 0; t < 8; ++t) red[wv][t][lane] = live ? acc[t] : floatx4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    floatx4 x = red[0][t][lane];
#pragma unroll
    for (int u = 1; u < kProxyGroup; ++u) x += red[u][t][lane];
    acc[t] = x;
  }
  // lane (i, j) holds batch rows 4j .. 4j+3 of columns n0 + 8i + t
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int b = 4 * j + e;
    if (b < B) {
      float* dst = partial + ((int64_t)blockIdx.y * B + b) * n_out + n0 + 8 * i;
      *(floatx4*)dst = floatx4{acc[0][e], acc[1][e], acc[2][e], acc[3][e]};
      *(floatx4*)(dst + 4) = floatx4{acc[4][e], acc[5][e], acc[6][e], acc[7][e]};
    }
  }
}

// Adds the row splits in split order.  Each thread's splits are loaded 32 at a
// time with straight-line loads (indices clamped, extra copies masked), so a
// d_model of 4096 costs one memory round trip instead of one per few splits.
__global__ __launch_bounds__(256) void proxy_reduce_kernel(const float* partial, int splits,
                                                           int total, float* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  constexpr int SB = 32;
  float s = 0.f;
  for (int k0 = 0; k0 < splits; k0 += SB) {
    float v[SB];
#pragma unroll
    for (int k = 0; k < SB; ++k) v[k] = partial[(int64_t)min(k0 + k, splits - 1) * total + i];
#pragma unroll
    for (int k = 0; k < SB; ++k)
      if (k0 + k < splits) s += v[k];
  }
  out[i] = s;
}

int proxy_splits(int d_model) { return (d_model / kProxyRows + kProxyGroup - 1) / kProxyGroup; }

kap_status launch_proxy(const uint16_t* hidden, const uint16_t* wq, int32_t B, int32_t dm,
                        int32_t n_out, float* q_out, float* partial, int32_t splits,
                        hipStream_t stream) {
  hipLaunchKernelGGL(proxy_mfma_kernel, dim3(n_out / kProxyMfmaCols, splits), dim3(64 * kProxyGroup), 0, stream,
                     hidden, wq, B, dm, n_out, partial);
  kap_status st = check_launch("proxy partial");
  if (st != KAP_OK) return st;
  const int total = B * n_out;
  hipLaunchKernelGGL(proxy_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, stream,
                     partial, splits, total, q_out);
  return check_launch("proxy reduce");
}

}  // namespace kap
