// KV copies on the path, both bit for bit:
//  * append through a slot mapping ([KAP] verifier: a verify pass moves the
//    committed full-context KV forward; [KAP] selected-KV view: the slot
//    mapping gives each new token its physical page and offset);
//  * compact workspace materialization ([KAP] selected-KV view: the executor
//    materializes a compact physical view; shape stabilization: a reusable
//    compact KV workspace).
//
// Append: one block per new token (b, i).  The token's K rows (Hkv x D,
// contiguous in the input) land in one token row per KV head of the
// token-major K page, so consecutive threads write consecutive dims.  V is
// dim-major inside a page: the token's value of dim d goes to column `offset`
// of row d, so its writes are strided by the page size.  A few KiB per token;
// latency-bound.
//
// Materialize: one block per (workspace page (b, j), KV head g).  Head slot g
// of workspace page b*cap + j receives head g of compact page j of row
// (b, G == 1 ? 0 : g): its K tile and V tile (16*D elements each) move as
// 16-byte words, every thread's loads issued before its stores.  HBM-bound: 2 x 2 x 16 x D x eb
// bytes (read + write, K and V) per (selected page, KV head).
#include "kap_internal.h"

namespace kap {

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  const int64_t* slot;
  int32_t Hkv, D;
  int64_t num_slots;
  void* k;
  void* v;
};

template <typename T>
__global__ __launch_bounds__(256) void append_kv_kernel(AppendArgs a) {
  const int64_t tok = blockIdx.x;  // b * q_new + i
  const int64_t s = a.slot[tok];
  if (s < 0 || s >= a.num_slots) return;
  const int64_t page = s / kPage;
  const int off = (int)(s % kPage);
  const int n = a.Hkv * a.D;
  const T* kn = (const T*)a.k_new + tok * n;
  const T* vn = (const T*)a.v_new + tok * n;
  T* k = (T*)a.k;
  T* v = (T*)a.v;
  for (int e = threadIdx.x; e < n; e += 256) {
    const int64_t g = e / a.D, d = e % a.D;
    k[((page * a.Hkv + g) * kPage + off) * a.D + d] = kn[e];
    v[((page * a.Hkv + g) * a.D + d) * kPage + off] = vn[e];
  }
}

kap_status launch_append(const void* k_new, const void* v_new, kap_dtype dt, const int64_t* slot,
                         int32_t B, int32_t q_new, int32_t Hkv, int32_t D, int64_t num_slots,
                         void* k, void* v, hipStream_t stream) {
  AppendArgs a{k_new, v_new, slot, Hkv, D, num_slots, k, v};
  const dim3 grid((unsigned)((int64_t)B * q_new));
  if (dt == KAP_BF16) hipLaunchKernelGGL(append_kv_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(append_kv_kernel<float>, grid, dim3(256), 0, stream, a);
  return check_launch("append kv");
}

struct MaterializeArgs {
  const uint4* k;
  const uint4* v;
  const int32_t* cbt;
  int32_t Hkv, G, cap;
  int32_t tile;  // 16-byte words per (page, head) K or V tile
  uint4* kws;
  uint4* vws;
  int32_t* ws_table;
};

__global__ __launch_bounds__(256) void materialize_kernel(MaterializeArgs a) {
  const int j = blockIdx.x, b = blockIdx.y, g = blockIdx.z;
  const int64_t dst = (int64_t)b * a.cap + j;
  if (g == 0 && threadIdx.x < a.G) {
    const int64_t t = ((int64_t)b * a.G + threadIdx.x) * a.cap + j;
    a.ws_table[t] = a.cbt[t] >= 0 ? (int32_t)dst : -1;
  }
  const int32_t src = a.cbt[((int64_t)b * a.G + (a.G == 1 ? 0 : g)) * a.cap + j];
  if (src < 0) return;
  const uint4* ks = a.k + ((int64_t)src * a.Hkv + g) * a.tile;
  const uint4* vs = a.v + ((int64_t)src * a.Hkv + g) * a.tile;
  uint4* kd = a.kws + (dst * a.Hkv + g) * a.tile;
  uint4* vd = a.vws + (dst * a.Hkv + g) * a.tile;
  constexpr int U = 2;  // words per thread in flight (a bf16 D = 128 tile is 256 words)
  // source tiles are read once: streaming loads
  for (int w0 = threadIdx.x; w0 < a.tile; w0 += 256 * U) {
    uint4 kw[U], vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = w0 + u * 256;
      if (w < a.tile) {
        kw[u] = ld_stream16(ks + w);
        vw[u] = ld_stream16(vs + w);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int w = w0 + u * 256;
      if (w < a.tile) {
        kd[w] = kw[u];
        vd[w] = vw[u];
      }
    }
  }
}

kap_status launch_materialize(const void* k, const void* v, kap_dtype dt, int32_t Hkv, int32_t D,
                              const int32_t* cbt, int32_t B, int32_t G, int32_t cap, void* kws,
                              void* vws, int32_t* ws_table, hipStream_t stream) {
  const int eb = dt == KAP_BF16 ? 2 : 4;
  MaterializeArgs a{(const uint4*)k, (const uint4*)v, cbt, Hkv, G, cap, kPage * D * eb / 16,
                    (uint4*)kws, (uint4*)vws, ws_table};
  hipLaunchKernelGGL(materialize_kernel, dim3(cap, B, Hkv), dim3(256), 0, stream, a);
  return check_launch("materialize");
}

}  // namespace kap
