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
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

#define GP_WAVE 64
#define GP_LOG2E 1.4426950408889634f
#define GP_LN2 0.6931471805599453f

namespace gp {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Load of data read once per launch (K/V pages in decode): a nontemporal load, which marks the
// lines as streaming. On MI355X a read-only stream of random 32 KB pages reaches ~6.2 TB/s with
// ordinary loads and ~7.0 TB/s with these when every instruction reads whole 128-byte lines;
// when an instruction reads only half of each line, these are slower than ordinary loads.
template <typename T>
__device__ __forceinline__ T ld_stream(const void* ptr) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(ptr));
}

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

// Signed 4-bit codes (two's complement nibbles) -> exact half values. A code c becomes the
// biased nibble u = c + 8 (= nibble ^ 8); placed in the low mantissa bits of 1024.0 (0x6400,
// whose half spacing is 1) it reads as 1024 + u, and subtracting 1032 leaves c exactly. A
// nibble in bits 4..7 of a half reads as 1024 + 16u; times 1/16 minus 72 it is c again.
__device__ __forceinline__ f16x2_t int4_lo_pair(uint32_t x) {  // nibbles at bits 0..3, 16..19
  return __builtin_bit_cast(f16x2_t, (x & 0x000F000Fu) ^ 0x64086408u) - f16x2_t{1032, 1032};
}
__device__ __forceinline__ f16x2_t int4_hi_pair(uint32_t x) {  // nibbles at bits 4..7, 20..23
  return __builtin_bit_cast(f16x2_t, (x & 0x00F000F0u) ^ 0x64806480u) * f16x2_t{0.0625, 0.0625} -
         f16x2_t{72, 72};
}

// Eight codes of one dword (nibble j = element j) -> halves in the element order
// (0, 4, 1, 5, 2, 6, 3, 7).
__device__ __forceinline__ f16x8_t int4x8_to_f16x8(uint32_t w) {
  const f16x2_t a = int4_lo_pair(w), b = int4_hi_pair(w);
  const f16x2_t c = int4_lo_pair(w >> 8), d = int4_hi_pair(w >> 8);
  return f16x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Four codes in the low 16 bits (nibble j = element j) -> halves in the order (0, 2, 1, 3).
__device__ __forceinline__ f16x4_t int4x4_to_f16x4(uint32_t w) {
  const uint32_t x = (w & 0xffu) | ((w & 0xff00u) << 8);  // byte 1 moves to byte 2
  const f16x2_t a = int4_lo_pair(x), b = int4_hi_pair(x);
  return f16x4_t{a.x, a.y, b.x, b.y};
}

// One word of two 4-code groups (dimension A in bits 0..15, dimension B in 16..31; nibble j of a
// group = token j) -> the halves of both dimensions, each in the token order (0, 2, 1, 3). One
// byte permute first interleaves the groups' bytes (A.b0, B.b0, A.b1, B.b1), so that each mask
// picks two tokens of one dimension and a single shift serves dimension B.
__device__ __forceinline__ void int4_word_to_f16x4x2(uint32_t w, f16x4_t& a, f16x4_t& b) {
  const uint32_t x = __builtin_amdgcn_perm(w, w, 0x03010200u);
  const f16x2_t a02 = int4_lo_pair(x), a13 = int4_hi_pair(x);
  const f16x2_t b02 = int4_lo_pair(x >> 8), b13 = int4_hi_pair(x >> 8);
  a = f16x4_t{a02.x, a02.y, a13.x, a13.y};
  b = f16x4_t{b02.x, b02.y, b13.x, b13.y};
}

__device__ __forceinline__ float half_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float half_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// x times the half in the low / high 16 bits of w, rounded once to float: written as an fma with
// a +0 addend of the widened half so that it becomes one mixed-precision fma instruction instead of
// a conversion and a product (same value; only a -0 product turns into +0).
__device__ __forceinline__ float mul_half_lo(float x, uint32_t w) {
  return __builtin_fmaf(x, (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)), 0.0f);
}
__device__ __forceinline__ float mul_half_hi(float x, uint32_t w) {
  return __builtin_fmaf(x, (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)), 0.0f);
}

// Dual-timescale EMA step (GrowPage Sec. 3.2 Eq. 6) on four consecutive elements of one slot's
// short and long summaries: x <- beta_x * x + (1 - beta_x) * q, or x = q on the slot's first step.
// Shared by the standalone update and the one fused into decode attention, so both give the
// same bits.
__device__ __forceinline__ void ema_update4(float* short_row, float* long_row, const float q[4],
                                            bool fresh, float beta_s, float beta_l) {
  f32x4_t* s = reinterpret_cast<f32x4_t*>(short_row);
  f32x4_t* l = reinterpret_cast<f32x4_t*>(long_row);
  if (fresh) {
    const f32x4_t v = {q[0], q[1], q[2], q[3]};
    *s = v;
    *l = v;
  } else {
    f32x4_t vs = *s, vl = *l;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      vs[c] = beta_s * vs[c] + (1.0f - beta_s) * q[c];
      vl[c] = beta_l * vl[c] + (1.0f - beta_l) * q[c];
    }
    *s = vs;
    *l = vl;
  }
}

// Four consecutive query elements as fp32 (bf16 or fp32 storage).
template <bool BF16>
__device__ __forceinline__ void load_q4(const void* q, size_t idx, float x[4]) {
  if constexpr (BF16) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(q) + idx);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const f32x4_t w = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(q) + idx);
    x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
  }
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

// exp2 that maps -inf to 0 without producing NaN for (-inf) - (-inf). The hardware exp2
// (v_exp_f32, about 1 ulp; results below 2^-126 flush to zero, which a softmax weight can
// afford) instead of the library's denormal-preserving expansion.
__device__ __forceinline__ float safe_exp2_diff(float a, float m) {
  return (a == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(a - m);
}

__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16_16x16x16(i16x4_t a, i16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16_16x16x32(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f16_16x16x16(f16x4_t a, f16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32_16x16x4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace gp

#define GP_CHECK_LAUNCH()                                 \
  do {                                                    \
    if (hipGetLastError() != hipSuccess) return GP_ERR_HIP; \
  } while (0)

// Wave64 reductions on the data-parallel-primitive (DPP) path: lane permutations inside rows
// of 16 (quad swaps, half-row and row mirrors), then the row broadcasts of lanes 15 and 31,
// leave the full reduction in lane 63, which is read back as a wave-uniform value. Unlike
// __shfl_xor these never go through the LDS permute unit.
namespace gp {

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane63_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror, row_bcast:15,
// row_bcast:31 (the broadcasts only update rows 1,3 and 2,3 respectively).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v += dpp_u64<0xb1>(v);
  v += dpp_u64<0x4e>(v);
  v += dpp_u64<0x141>(v);
  v += dpp_u64<0x140>(v);
  v += dpp_u64<0x142, 0xa>(v);
  v += dpp_u64<0x143, 0xc>(v);
  return readlane63_u64(v);
}

__device__ __forceinline__ double wave_sum_f64(double x) {
  uint64_t v = __builtin_bit_cast(uint64_t, x);
  x += __builtin_bit_cast(double, dpp_u64<0xb1>(v));
  v = __builtin_bit_cast(uint64_t, x);
  x += __builtin_bit_cast(double, dpp_u64<0x4e>(v));
  v = __builtin_bit_cast(uint64_t, x);
  x += __builtin_bit_cast(double, dpp_u64<0x141>(v));
  v = __builtin_bit_cast(uint64_t, x);
  x += __builtin_bit_cast(double, dpp_u64<0x140>(v));
  v = __builtin_bit_cast(uint64_t, x);
  x += __builtin_bit_cast(double, dpp_u64<0x142, 0xa>(v));
  v = __builtin_bit_cast(uint64_t, x);
  x += __builtin_bit_cast(double, dpp_u64<0x143, 0xc>(v));
  return __builtin_bit_cast(double, readlane63_u64(__builtin_bit_cast(uint64_t, x)));
}

// Maximum with the lane 16 (or 32) positions away: gfx950's lane-swap instructions exchange the
// odd and even rows of a wave (or its two halves) in the VALU, without the LDS permute path.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wave-uniform copies of values that every lane holds alike (a reduction result, a broadcast from
// LDS, a field of a record all lanes loaded): kept in scalar registers, so that the branches and
// loops they control are scalar, not masked per lane.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t uni(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ uint64_t uni(uint64_t v) {
  const uint32_t lo = uni((uint32_t)v), hi = uni((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double uni(double v) {
  return __builtin_bit_cast(double, uni(__builtin_bit_cast(uint64_t, v)));
}

// Larger and smaller of this lane's value and lane (lane ^ J)'s: quad permutations fetch the
// partner for 1 and 2; for 4 and 8 a quad reversal (lane ^ 3) or half-row mirror (lane ^ 7 in an
// 8-lane half) followed by the half-row (7 - i) or row (15 - i) mirror; for 16 and 32 the
// lane-swap instructions leave the two values of each pair in the two results.
template <int J>
__device__ __forceinline__ void lane_pair_minmax(uint32_t v, uint32_t& hi, uint32_t& lo) {
  static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "lane_pair_minmax: J");
  uint32_t a = v, b;
  if constexpr (J == 1) b = dpp_u32<0xb1>(v);
  if constexpr (J == 2) b = dpp_u32<0x4e>(v);
  if constexpr (J == 4) b = dpp_u32<0x141>(dpp_u32<0x1b>(v));
  if constexpr (J == 8) b = dpp_u32<0x140>(dpp_u32<0x141>(v));
  if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
  if constexpr (J == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0];
    b = r[1];
  }
  hi = max(a, b);
  lo = min(a, b);
}

// Inclusive prefix sum over the 64 lanes (lane order): shifts by 1, 2, 4 and 8 inside each row of
// 16, then the row broadcasts of lanes 15 and 31 carry the rows below.
__device__ __forceinline__ double wave_scan_f64(double x) {
  x += __builtin_bit_cast(double, dpp_u64<0x111>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x112>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x114>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x118>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x142, 0xa>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x143, 0xc>(__builtin_bit_cast(uint64_t, x)));
  return x;
}

// Inclusive prefix sum of 64-bit integers over the 64 lanes (lane order), as wave_scan_f64.
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t x) {
  x += dpp_u64<0x111>(x);
  x += dpp_u64<0x112>(x);
  x += dpp_u64<0x114>(x);
  x += dpp_u64<0x118>(x);
  x += dpp_u64<0x142, 0xa>(x);
  x += dpp_u64<0x143, 0xc>(x);
  return x;
}

// Sums and maxima over the 16 lanes of each DPP row (quad swaps, half-row and row mirrors): every
// lane of a row ends with its row's result. A block reduction hands its (at most 16) wave
// partials to the lanes of a row this way: one LDS read per lane instead of 16.
__device__ __forceinline__ double row16_sum_f64(double x) {
  x += __builtin_bit_cast(double, dpp_u64<0xb1>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x4e>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x141>(__builtin_bit_cast(uint64_t, x)));
  x += __builtin_bit_cast(double, dpp_u64<0x140>(__builtin_bit_cast(uint64_t, x)));
  return x;
}

__device__ __forceinline__ uint64_t row16_sum_u64(uint64_t v) {
  v += dpp_u64<0xb1>(v);
  v += dpp_u64<0x4e>(v);
  v += dpp_u64<0x141>(v);
  v += dpp_u64<0x140>(v);
  return v;
}

__device__ __forceinline__ uint32_t row16_sum_u32(uint32_t v) {
  v += dpp_u32<0xb1>(v);
  v += dpp_u32<0x4e>(v);
  v += dpp_u32<0x141>(v);
  v += dpp_u32<0x140>(v);
  return v;
}

// sum of unsigned values (lanes outside a broadcast's row mask add 0)
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += dpp_u32<0xb1>(v);
  v += dpp_u32<0x4e>(v);
  v += dpp_u32<0x141>(v);
  v += dpp_u32<0x140>(v);
  v += dpp_u32<0x142, 0xa>(v);
  v += dpp_u32<0x143, 0xc>(v);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xb1>(v));
  v = max(v, dpp_u32<0x4e>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  return v;
}

// maximum of unsigned values (lanes outside a broadcast's row mask see 0, the identity)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xb1>(v));
  v = max(v, dpp_u32<0x4e>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  v = max(v, dpp_u32<0x142, 0xa>(v));
  v = max(v, dpp_u32<0x143, 0xc>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace gp
