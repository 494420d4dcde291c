// Internal declarations shared by the libkap HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kap.h"

namespace kap {

// ---------------------------------------------------------------- constants
constexpr int kPage = 16;            // tokens per KV page
constexpr int kTargetItems = 1280;   // split-K work items aimed at per call (measured best at 128K, B = 4)
constexpr int kMinChunk = 2;         // minimum pages per work item
constexpr int kPipelinedMaxPages = 32;  // items up to this many pages run the pipelined kernel
constexpr int kMaxSelectPages = 65536;
constexpr int kMaxPlanRows = 4096;      // batch x KV heads per attention call

// ---------------------------------------------------------------- device types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __uint_as_float(((uint32_t)x) << 16);
}

// round-to-nearest-even, NaN kept quiet
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (low half = a), one round-to-nearest-even
// conversion instruction on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const float2v x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
}

template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// sin and cos of pos * inv_freq, both fp64.  The angle reaches ~1.3e5 rad at
// 128K context, so it is first reduced by 2*pi (split in two parts, Cody-Waite)
// to keep the library call on its small-argument path.
__device__ __forceinline__ void rope_sincos(double pos, int pair, int D, double log2_theta,
                                            double* s, double* c) {
  const double inv_freq = exp2(-(2.0 * pair / D) * log2_theta);
  const double ang = pos * inv_freq;
  const double k = rint(ang * 0.15915494309189535);       // 1 / (2 pi)
  double r = fma(-k, 6.283185307179586, ang);             // 2 pi, high part
  r = fma(-k, 2.4492935982947064e-16, r);                 // 2 pi, low part
  sincos(r, s, c);
}

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight across it (__syncthreads also waits for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max_xor(float v, int from, int to) {
  for (int m = from; m < to; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...);
kap_status fail(kap_status s, const char* fmt, ...);
kap_status check_launch(const char* what);
int resident_blocks(const void* kernel, int block_threads);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace carving for the attention calls (decode and verify share it).
struct AttnWorkspace {
  int32_t* n_items;     // [1]
  int32_t* row_off;     // [B*Hkv + 1] first work item of each (b, g)
  float2* part_ml;      // [max_items][R] (reference max in log2 units, sum)
  float* part_o;        // [max_items][R][D]
  int32_t max_items;
  size_t bytes;
};
AttnWorkspace carve_attn_workspace(void* base, int32_t B, int32_t q_len, int32_t Hq,
                                   int32_t Hkv, int32_t D);

struct AttnCall {
  const void* q;
  kap_dtype dtype;
  const int32_t* positions;
  int32_t q_len;
  float theta, scale;
  const void* k;
  const void* v;
  int32_t Hkv, D;
  const int32_t* table;
  int32_t width, G;
  const int32_t* lens;
  int32_t B, Hq;
  void* out;
  float* lse;
  AttnWorkspace ws;
  hipStream_t stream;
};
kap_status launch_attention(const AttnCall& c);

kap_status launch_score(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                        const void* summ, kap_dtype s_dt, const int32_t* bt, int32_t max_pages,
                        const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                        float* scores, hipStream_t stream);
// All KV heads per block plus the head-pooled key (scores may be null); Hkv <= 16.
kap_status launch_score_pool(const void* q, kap_dtype q_dt, const int32_t* pos, float theta,
                             const void* summ, kap_dtype s_dt, const int32_t* bt,
                             int32_t max_pages, const int32_t* seq_lens, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t D, float* scores, float* pooled,
                             hipStream_t stream);
kap_status launch_select(const float* scores, int32_t B, int32_t Hkv, int32_t max_pages,
                         const int32_t* seq_lens, int32_t per_head, const int32_t* anchor,
                         const int32_t* recent, const int32_t* k_mid, int32_t capacity,
                         int32_t* sel, int32_t* cnt, hipStream_t stream,
                         const int32_t* bt = nullptr, const int32_t* pos = nullptr,
                         int32_t q_new = 0, int32_t* cbt = nullptr, int32_t* clen = nullptr,
                         int64_t* slot = nullptr);
kap_status launch_compact(const int32_t* sel, const int32_t* cnt, int32_t B, int32_t G,
                          int32_t cap, const int32_t* bt, int32_t max_pages,
                          const int32_t* seq_lens, const int32_t* pos, int32_t q_new,
                          int32_t* cbt, int32_t* clog, int32_t* clen, int64_t* slot,
                          hipStream_t stream);
// first_pos == nullptr: every logical page; else only the pages holding
// tokens first_pos[b] .. first_pos[b] + q_new - 1.
kap_status launch_summary(const void* k, kap_dtype kv_dt, int32_t Hkv, int32_t D,
                          const int32_t* bt, int32_t max_pages, const int32_t* seq_lens,
                          const int32_t* first_pos, int32_t q_new, int32_t B, void* summ,
                          kap_dtype s_dt, hipStream_t stream);
kap_status launch_materialize(const void* k, const void* v, kap_dtype dt, int32_t Hkv, int32_t D,
                              const int32_t* cbt, int32_t B, int32_t G, int32_t cap, void* kws,
                              void* vws, int32_t* ws_table, hipStream_t stream);
kap_status launch_append(const void* k_new, const void* v_new, kap_dtype dt, const int64_t* slot,
                         int32_t B, int32_t q_new, int32_t Hkv, int32_t D, int64_t num_slots,
                         void* k, void* v, hipStream_t stream);
int proxy_splits(int d_model);
kap_status launch_diag_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);
kap_status launch_proxy(const uint16_t* hidden, const uint16_t* wq, int32_t B, int32_t dm,
                        int32_t n_out, float* q_out, float* partial, int32_t splits,
                        hipStream_t stream);

}  // namespace kap
