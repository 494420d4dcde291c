// Proxy query for early routing (EarlySelectKV news item, Interpretation: the
// side flow projects a preceding hidden state through the query projection to
// obtain the routing query).  q_out = hidden @ W_q, bf16 inputs, fp32 sums.
//
// HBM-bound GEMV (B <= 16 rows share each W_q byte).  Block (256 threads)
// owns 64 output columns x 512 rows of W_q: 8 lanes cover one 128-byte row
// segment with 16-byte loads, so one wave-wide load reads 8 full rows.
// Each lane accumulates B x 8 columns over its rows; partial sums are
// reduced inside the block in a fixed order and written per row split, and a
// second small kernel adds the splits in split order (deterministic).
#include "kap_internal.h"

namespace kap {

constexpr int kProxyCols = 64;
constexpr int kProxyRows = 512;

template <int BM>
__global__ __launch_bounds__(256) void proxy_partial_kernel(const uint16_t* hidden,
                                                            const uint16_t* wq, int B, int dm,
                                                            int n_out, float* partial) {
  const int n0 = blockIdx.x * kProxyCols;
  const int split = blockIdx.y;
  const int c0 = split * kProxyRows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int part = lane & 7, rsub = lane >> 3;
  __shared__ float sh[BM][kProxyRows];
  for (int e = tid; e < BM * kProxyRows; e += 256) {
    const int b = e / kProxyRows, c = e % kProxyRows;
    sh[b][c] = (b < B) ? bf16_to_f32(hidden[(int64_t)b * dm + c0 + c]) : 0.f;
  }
  __syncthreads();
  float acc[BM][8];
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[b][e] = 0.f;
  const uint16_t* wbase = wq + (int64_t)c0 * n_out + n0 + part * 8;
  for (int r = wave * 8 + rsub; r < kProxyRows; r += 32) {
    const uint4 w = *(const uint4*)(wbase + (int64_t)r * n_out);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float wf[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wf[2 * e] = __uint_as_float(ww[e] << 16);
      wf[2 * e + 1] = __uint_as_float(ww[e] & 0xffff0000u);
    }
#pragma unroll
    for (int b = 0; b < BM; ++b) {
      const float h = sh[b][r];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[b][e] += h * wf[e];
    }
  }
  // lanes with the same `part` differ in bits 3..5: butterfly over them
  __shared__ float red[4][BM][kProxyCols];
#pragma unroll
  for (int b = 0; b < BM; ++b)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[b][e];
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (rsub == 0) red[wave][b][part * 8 + e] = v;
    }
  __syncthreads();
  for (int e = tid; e < BM * kProxyCols; e += 256) {
    const int b = e / kProxyCols, col = e % kProxyCols;
    if (b < B) {
      const float s = ((red[0][b][col] + red[1][b][col]) + red[2][b][col]) + red[3][b][col];
      partial[((int64_t)split * B + b) * n_out + n0 + col] = s;
    }
  }
}

__global__ __launch_bounds__(256) void proxy_reduce_kernel(const float* partial, int splits,
                                                           int total, float* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += partial[(int64_t)k * total + i];
  out[i] = s;
}

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
