// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, wave-wide
// reductions over 64 lanes, vector types, launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // raw bf16 storage
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even float -> bf16 (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<bf16_t>((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// Two floats -> packed bf16 pair (low half = a), round-to-nearest-even, one
// v_cvt_pk_bf16_f32 on gfx950.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 r = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = __shfl_xor(v, m, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Order-preserving map of a finite float to uint32 (larger float -> larger integer),
// with -0.0 folded onto +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Standard normal cdf, Phi(z) = erfc(-z / sqrt 2) / 2, with erfc from Abramowitz and
// Stegun, Handbook of Mathematical Functions, formula 7.1.26: for x >= 0,
// erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2), t = 1 / (1 + p x),
// absolute error at most 1.5e-7. Branch-free (one reciprocal, one exponential), so a
// GEMM epilogue applying it to every output costs a few instructions per value.
__device__ __forceinline__ float normal_cdf(float z) {
  const float ax = fabsf(z) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  const float poly =
      t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                       -0.284496736f),
               0.254829592f);
  const float half_erfc = 0.5f * poly * __expf(-ax * ax);
  return z >= 0.f ? 1.0f - half_erfc : half_erfc;
}

// GELU with the exact (erf) form: z Phi(z).
__device__ __forceinline__ float gelu_erf(float z) {
  return z * normal_cdf(z);
}

// z sigma(z), with the hardware reciprocal (1 ulp) in place of a rounded division: a
// SwiGLU epilogue evaluates it once per output.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe

// Kernel profiling hooks (host side, see moe_profile_enable).
namespace moe_prof {
void before(const char* name, hipStream_t s);
void after(const char* name, hipStream_t s);
}  // namespace moe_prof

#define MOE_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                   \
  do {                                                                              \
    moe_prof::before(name, stream);                                                 \
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);            \
    if (hipGetLastError() != hipSuccess) return MOE_ERR_HIP;                        \
    moe_prof::after(name, stream);                                                  \
  } while (0)
