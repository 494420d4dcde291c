// Device-side constants, types and helpers shared by the libkap kernels
// (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kap.h"

namespace kap {

// ---------------------------------------------------------------- constants
constexpr int kPage = 16;            // tokens per KV page
constexpr int kTargetItems = 1280;   // split-K work items aimed at per call (measured best at 128K, B = 4)
constexpr int kMinChunk = 2;         // minimum pages per work item
constexpr int kShortItemPages = 32;  // items up to this many pages run the pair loop
constexpr int kPairs2MinPages = 8;   // one-tile items this long keep two pairs in flight
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

// sin and cos of one position step for pair `pair` (the angle rope_sincos
// advances by per position), for angle-addition steps between positions.
__device__ __forceinline__ void rope_step(int pair, int D, double log2_theta, double* s, double* c) {
  const double inv_freq = exp2(-(2.0 * pair / D) * log2_theta);
  sincos(inv_freq, s, c);
}

// Streaming loads with the non-temporal policy, which marks the lines for
// early eviction instead of keeping them cached.  On MI355X it raises the
// sustained read rate of a plain stream from about 6.3 to 7.2 TB/s, and of
// random 8 KiB page tiles by about 10 %, when every load covers whole 128-byte
// lines.  For data a call reads once; not for page tables or queries.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
  const u32x4v v = __builtin_nontemporal_load((const u32x4v*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const void* p) {
  const u32x2v v = __builtin_nontemporal_load((const u32x2v*)p);
  return make_uint2(v.x, v.y);
}

// Wave-wide integer prefix sums and reductions on DPP lane moves (row shifts
// within each 16-lane row, then row broadcasts), a few VALU cycles per step
// instead of an LDS round trip per step for shuffles.  Inclusive scan over the
// 64 lanes in lane order; the total is lane 63's value.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}
__device__ __forceinline__ int wave_sum(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}
// maximum over the wave of values >= 0 (0 is the identity of the steps)
__device__ __forceinline__ int wave_max_nonneg(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight across it (__syncthreads also waits for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Max and sum over the four lanes i, i ^ 16, i ^ 32, i ^ 48 (the same lane of
// each 16-lane row) with gfx950's row-swap moves (one VALU instruction per
// exchange).  The sum adds in the order (x_i + x_{i^16}) + (x_{i^32} + x_{i^48})
// for every lane, as an xor butterfly does.
__device__ __forceinline__ void rows_exchange16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void rows_exchange32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float rows_max(float v) {
  float a, b;
  rows_exchange16(v, a, b);
  rows_exchange32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum(float v) {
  float a, b;
  rows_exchange16(v, a, b);
  rows_exchange32(a + b, a, b);
  return a + b;
}

}  // namespace kap
