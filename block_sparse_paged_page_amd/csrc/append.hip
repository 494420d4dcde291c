// KV append through a slot mapping ([KAP] verifier: verification advances the
// committed full-context KV state; [KAP] selected-KV view: slot mappings place
// newly scheduled tokens into their physical KV slots).
//
// One block per new token (b, i).  The token's K rows (Hkv x D, contiguous in
// the input) land in one token row per KV head of the token-major K page, so
// consecutive threads write consecutive dims.  V is dim-major inside a page:
// the token's value of dim d goes to column `offset` of row d, so its writes
// are strided by the page size.  A few KiB per token; latency-bound.
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

}  // namespace kap
