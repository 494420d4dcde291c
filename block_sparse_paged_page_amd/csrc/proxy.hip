// Proxy query for early routing (EarlySelectKV news item, Interpretation: the
// side flow projects a preceding hidden state through the query projection to
// obtain the routing query).  q_out = hidden @ W_q, bf16 inputs, fp32 sums.
//
// HBM-bound GEMV (B <= 16 rows share each W_q byte).  A block (4 waves) owns a
// tile of 256 output columns x kProxyRows rows of W_q; every wave-wide load
// reads 512 B of one W_q row contiguously (lane l: columns 4l .. 4l+3), and a
// wave keeps all 32 of its rows in flight.  Each lane accumulates B x 4
// columns over its rows; the four waves are added in wave order through LDS and each row split
// writes its partial sums; a second kernel adds the splits in split order
// (deterministic).
#include "kap_internal.h"

namespace kap {

constexpr int kProxyCols = 256;  // columns per block: 64 lanes x 4
constexpr int kProxyRows = 128;  // W_q rows per block (32 per wave)

template <int BM>
__global__ __launch_bounds__(256) void proxy_partial_kernel(const uint16_t* hidden,
                                                            const uint16_t* wq, int B, int dm,
                                                            int n_out, float* partial) {
  const int n0 = blockIdx.x * kProxyCols;
  const int split = blockIdx.y;
  const int c0 = split * kProxyRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int RPW = kProxyRows / 4;  // rows per wave
  // rows in flight at once: all of the wave's rows, or 16 when the batch is 16
  constexpr int INFL = BM >= 16 ? 16 : RPW;
  const uint16_t* wbase = wq + (int64_t)(c0 + wave * RPW) * n_out + n0 + lane * 4;
  // The hidden-state slice is requested first and the W_q rows right after.
  // Loads complete in issue order, so staging the slice in LDS waits only for
  // its own few loads, and the row loop below waits for one W_q row at a time:
  // each row's FMAs run while the later rows are still in flight.  (Issued the
  // other way round, staging the slice waited for every W_q row, and all of
  // the arithmetic ran after the whole burst had arrived.)  W_q is read once
  // per call: streaming loads.
  __shared__ float sh[BM][kProxyRows];
  constexpr int PER = BM * kProxyRows / 256 > 0 ? BM * kProxyRows / 256 : 1;  // values per thread
  uint16_t hraw[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = k * 256 + tid;
    const int b = e / kProxyRows, c = e % kProxyRows;
    hraw[k] = hidden[(int64_t)min(b, B - 1) * dm + c0 + c];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the slice's loads ahead of the rows
  uint2 wrow[INFL];
#pragma unroll
  for (int r = 0; r < INFL; ++r) wrow[r] = ld_stream8(wbase + (int64_t)r * n_out);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = k * 256 + tid;
    const int b = e / kProxyRows, c = e % kProxyRows;
    if (e < BM * kProxyRows) sh[b][c] = b < B ? bf16_to_f32(hraw[k]) : 0.f;
  }
  lds_barrier();
  float acc[BM][4];
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[b][e] = 0.f;
#pragma unroll
  for (int r0 = 0; r0 < RPW; r0 += INFL) {
    if (r0 > 0) {
#pragma unroll
      for (int r = 0; r < INFL; ++r)
        wrow[r] = ld_stream8(wbase + (int64_t)(r0 + r) * n_out);
    }
#pragma unroll
    for (int rr = 0; rr < INFL; ++rr) {
      const int r = r0 + rr;
      const uint32_t ww[2] = {wrow[rr].x, wrow[rr].y};
      float wf[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        wf[2 * e] = __uint_as_float(ww[e] << 16);
        wf[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
      }
#pragma unroll
      for (int b = 0; b < BM; ++b) {
        const float h = sh[b][wave * RPW + r];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[b][e] += h * wf[e];
      }
    }
  }
  // waves 1..3 hand their sums to wave 0 through LDS, added in wave order,
  // eight batch rows at a time
  constexpr int BC = BM < 8 ? BM : 8;
  __shared__ float red[3][BC][kProxyCols];
#pragma unroll
  for (int b0 = 0; b0 < BM; b0 += BC) {
    if (wave > 0) {
#pragma unroll
      for (int bb = 0; bb < BC; ++bb)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave - 1][bb][lane * 4 + e] = acc[b0 + bb][e];
    }
    lds_barrier();
    if (wave == 0) {
#pragma unroll
      for (int bb = 0; bb < BC; ++bb) {
        const int b = b0 + bb;
        if (b < B) {
          float* dst = partial + ((int64_t)split * B + b) * n_out + n0 + lane * 4;
          floatx4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = lane * 4 + e;
            o[e] = ((acc[b][e] + red[0][bb][col]) + red[1][bb][col]) + red[2][bb][col];
          }
          *(floatx4*)dst = o;
        }
      }
    }
    lds_barrier();
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

int proxy_splits(int d_model) { return d_model / kProxyRows; }

kap_status launch_proxy(const uint16_t* hidden, const uint16_t* wq, int32_t B, int32_t dm,
                        int32_t n_out, float* q_out, float* partial, int32_t splits,
                        hipStream_t stream) {
  dim3 grid(n_out / kProxyCols, splits);
#define KAP_PROXY(BM) \
  hipLaunchKernelGGL((proxy_partial_kernel<BM>), grid, dim3(256), 0, stream, hidden, wq, B, dm, \
                     n_out, partial)
  if (B <= 1) KAP_PROXY(1);
  else if (B <= 2) KAP_PROXY(2);
  else if (B <= 4) KAP_PROXY(4);
  else if (B <= 8) KAP_PROXY(8);
  else KAP_PROXY(16);
#undef KAP_PROXY
  kap_status st = check_launch("proxy partial");
  if (st != KAP_OK) return st;
  const int total = B * n_out;
  hipLaunchKernelGGL(proxy_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, stream,
                     partial, splits, total, q_out);
  return check_launch("proxy reduce");
}

}  // namespace kap
