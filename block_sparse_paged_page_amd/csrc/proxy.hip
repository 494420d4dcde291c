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

// ---------------------------------------------------------------- packed W_q
// The query projection is a static weight, so it can be re-laid once for the
// GEMV.  Packed layout, per 16-column tile ct, per 32-row step k32, per group
// kg of 8 rows, per column c: the 8 rows' values of column 16 ct + c, i.e.
//   wp[((((ct * (dm / 32) + k32) * 4 + kg) * 16 + c) * 8 + i] = wq[32 k32 + 8 kg + i][16 ct + c].
// A 16-byte group is exactly one lane's B operand of v_mfma_f32_16x16x32_bf16
// (lane kg * 16 + c: 8 consecutive k of column c), a wave's k-step is 1 KiB
// of contiguous bytes, and a column tile's whole d_model is one contiguous
// run.  So one block per 16 columns can stream its share with all of the
// chip's CUs busy and add its row splits in LDS: one launch, no partial sums
// through memory.  (The row-major kernel above needs 128-column tiles for
// 256-byte row segments, which leaves too few blocks per column tile to keep
// every split in one block.)
constexpr int kPackedWaves = 8;   // waves per column tile, each a contiguous share of the k-steps
constexpr int kPackedSteps = 16;  // k-steps a wave keeps in flight at once (512 rows of W_q)

__global__ __launch_bounds__(256) void proxy_pack_kernel(const uint16_t* wq, uint16_t* wp, int dm,
                                                         int n_out) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one 16-byte group
  if (o >= (int64_t)n_out * dm / 8) return;
  const int steps = dm / 32;
  const int c = (int)(o & 15), kg = (int)((o >> 4) & 3);
  const int64_t k32 = (o >> 6) % steps, ct = (o >> 6) / steps;
  const uint16_t* src = wq + (k32 * 32 + kg * 8) * n_out + ct * 16 + c;
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v[i] = (uint32_t)src[(int64_t)(2 * i) * n_out] | ((uint32_t)src[(int64_t)(2 * i + 1) * n_out] << 16);
  *(uint4*)(wp + o * 8) = make_uint4(v[0], v[1], v[2], v[3]);
}

// q_out = hidden @ W_q over the packed weight.  Block = one 16-column tile,
// kPackedWaves waves; wave w takes k-steps [w per, (w + 1) per) of the
// d_model / 32, per = ceil(steps / kPackedWaves), in rounds of kPackedSteps
// (a last partial round loads at clamped indices and masks the steps outside
// the wave's share to zero on both operands).  A = the hidden rows (M = B
// <= 16, rows past B zero), B operand = the packed groups.  The waves' sums
// are added in wave order through LDS (deterministic).
__global__ __launch_bounds__(64 * kPackedWaves) void proxy_packed_kernel(
    const uint16_t* hidden, const uint16_t* wp, int B, int dm, int n_out, float* q_out) {
  const int ct = blockIdx.x, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, kg = lane >> 4;
  const int steps = dm / 32;
  const int per = (steps + kPackedWaves - 1) / kPackedWaves;
  const int s0 = wv * per, s1 = min(s0 + per, steps);
  const uint16_t* wt = wp + ((int64_t)ct * steps * 64 + lane) * 8;
  const uint16_t* hrow = hidden + (int64_t)min(m, B - 1) * dm + kg * 8;
  const uint32_t row_keep = m < B ? 0xffffffffu : 0u;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = s0; r0 < s1; r0 += kPackedSteps) {
    if (r0 + kPackedSteps <= s1) {
      // a full round: fixed offsets, no masks.  Left to the compiler's
      // schedule, which keeps about half of the round's loads in flight:
      // 7.7 us per call for a 4096 x 4096 W_q at B = 8, against 8.6 us with
      // every load forced above the first MFMA.
      const uint16_t* wr = wt + 512 * (int64_t)r0;
      const uint16_t* hr = hrow + 32 * (int64_t)r0;
      uint4 hf[kPackedSteps], wf[kPackedSteps];
#pragma unroll
      for (int t = 0; t < kPackedSteps; ++t) hf[t] = *(const uint4*)(hr + 32 * t);
#pragma unroll
      for (int t = 0; t < kPackedSteps; ++t) wf[t] = ld_stream16(wr + 512 * t);  // read once per call
#pragma unroll
      for (int t = 0; t < kPackedSteps; ++t) {
        const uint4 h = make_uint4(hf[t].x & row_keep, hf[t].y & row_keep, hf[t].z & row_keep,
                                   hf[t].w & row_keep);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h),
                                                      __builtin_bit_cast(bf16x8, wf[t]), acc, 0, 0, 0);
      }
      continue;
    }
    // the share's last, partial round: clamped indices, masked steps
    uint4 hf[kPackedSteps], wf[kPackedSteps];
#pragma unroll
    for (int t = 0; t < kPackedSteps; ++t)
      hf[t] = *(const uint4*)(hrow + 32 * (int64_t)min(r0 + t, steps - 1));
#pragma unroll
    for (int t = 0; t < kPackedSteps; ++t)
      wf[t] = ld_stream16(wt + 512 * (int64_t)min(r0 + t, steps - 1));  // W_q is read once per call
    // every load above the first MFMA (the scheduler would otherwise sink
    // them next to their uses here and wait for each in turn)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < kPackedSteps; ++t) {
      const uint32_t in = r0 + t < s1 ? 0xffffffffu : 0u, hk = in & row_keep;
      const uint4 h = make_uint4(hf[t].x & hk, hf[t].y & hk, hf[t].z & hk, hf[t].w & hk);
      const uint4 w = make_uint4(wf[t].x & in, wf[t].y & in, wf[t].z & in, wf[t].w & in);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, h),
                                                    __builtin_bit_cast(bf16x8, w), acc, 0, 0, 0);
    }
  }
  __shared__ floatx4 red[kPackedWaves][64];
  red[wv][lane] = acc;
  __syncthreads();
  if (wv != 0) return;
  floatx4 x = red[0][lane];
#pragma unroll
  for (int u = 1; u < kPackedWaves; ++u) x += red[u][lane];
  // lane (m, kg) holds batch rows 4 kg .. 4 kg + 3 of column 16 ct + m
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int b = 4 * kg + e;
    if (b < B) q_out[(int64_t)b * n_out + ct * 16 + m] = x[e];
  }
}

kap_status launch_proxy_pack(const uint16_t* wq, uint16_t* wp, int32_t dm, int32_t n_out,
                             hipStream_t stream) {
  const int64_t groups = (int64_t)n_out * dm / 8;
  hipLaunchKernelGGL(proxy_pack_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0,
                     stream, wq, wp, dm, n_out);
  return check_launch("proxy weight pack");
}

kap_status launch_proxy_packed(const uint16_t* hidden, const uint16_t* wp, int32_t B, int32_t dm,
                               int32_t n_out, float* q_out, hipStream_t stream) {
  hipLaunchKernelGGL(proxy_packed_kernel, dim3(n_out / 16), dim3(64 * kPackedWaves), 0, stream,
                     hidden, wp, B, dm, n_out, q_out);
  return check_launch("proxy packed GEMV");
}

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
