// Device helpers shared by the gfx950 kernels: vector types, bf16/fp8 conversion, wave64
// reductions and the MFMA tile shapes used by the attention-style contractions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/growpage.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

#define GP_WAVE 64
#define GP_LOG2E 1.4426950408889634f
#define GP_LN2 0.6931471805599453f

namespace gp {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// round-to-nearest-even float -> bf16 bit pattern (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Four OCP E4M3FN codes (one dword, byte i = element i) -> four bf16 (exact: every E4M3
// value is representable in bf16). Uses the gfx950 fp8 -> f32 conversion.
__device__ __forceinline__ u32x2_t fp8x4_to_bf16x4(uint32_t codes) {
  f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
  f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
  u32x2_t r;
  r.x = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xffff0000u);
  r.y = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xffff0000u);
  return r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, GP_WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, GP_WAVE);
  return v;
}

// exp2 that maps -inf to 0 without producing NaN for (-inf) - (-inf)
__device__ __forceinline__ float safe_exp2_diff(float a, float m) {
  return (a == -INFINITY) ? 0.0f : exp2f(a - m);
}

__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32_16x16x4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace gp

#define GP_CHECK_LAUNCH()                                 \
  do {                                                    \
    if (hipGetLastError() != hipSuccess) return GP_ERR_HIP; \
  } while (0)
