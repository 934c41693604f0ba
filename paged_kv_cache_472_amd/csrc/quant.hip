// Demotion of bf16 pages to INT4 pages (PASK App. B.5, "Packed attention and quantization").
//
// One workgroup per listed page. Each thread owns one token row of one KV head: it reads the
// row's head_dim elements (a contiguous key row, and the value row gathered from the
// token-contiguous value block: consecutive threads read consecutive tokens), takes the largest
// magnitude, derives the half scale and writes the codes. Key codes pack along d (4 bytes per
// 8 elements); value codes pack along the token axis in four-token blocks with the dimensions
// interleaved (the layout the decode kernel reads with one 16-byte load per lane), so the
// even-token thread of each pair gathers its neighbour's codes with a lane shuffle and writes
// the shared bytes. The page tag
// changes last, after a barrier, so a reader of the tag never sees a half-written page.
//
// Exactness of the scale and codes against a float64 evaluation: the inputs are bf16 (8
// significant bits). amax / 7 in correctly rounded fp32 is at least 2^-14 relative away from
// every midpoint between half values unless it lies exactly on one (then fp32 holds it
// exactly), so rounding it to half in a second step gives the correctly rounded half. The code
// quotient x / s (correctly rounded fp32) is likewise at least 2^-12 away from every
// half-integer unless it is one exactly, so rounding it to an integer matches exact rounding.
#include "common.h"

namespace {

constexpr int QT_THREADS = 256;

struct QuantParams {
  const uint16_t* k;
  const uint16_t* v;
  uint8_t* k4;
  uint8_t* v4;
  uint16_t* k4_scale;
  uint16_t* v4_scale;
  uint8_t* page_tag;
  const int32_t* page_ids;
  int num_ids, num_pages, H_kv, b, D;
};

// Scale of a row with largest magnitude amax: half(amax / 7), at least 2^-24; 1 for a zero row.
__device__ __forceinline__ _Float16 row_scale(float amax) {
  if (amax == 0.f) return (_Float16)1.0f;
  const _Float16 h = (_Float16)__fdiv_rn(amax, 7.0f);  // round to nearest even
  const _Float16 tiny = __builtin_bit_cast(_Float16, (uint16_t)1);  // 2^-24
  return h < tiny ? tiny : h;
}

__device__ __forceinline__ uint32_t code_of(float x, float s) {
  float c = __builtin_rintf(__fdiv_rn(x, s));
  c = fminf(fmaxf(c, -7.f), 7.f);
  return (uint32_t)(int)c & 0xFu;
}

template <int D>
__global__ __launch_bounds__(QT_THREADS) void quantize_pages_kernel(QuantParams p) {
  const int pg = p.page_ids[blockIdx.x];
  if (pg < 0 || pg >= p.num_pages) return;
  if (p.page_tag[pg] != GP_TAG_BF16) return;  // uniform over the workgroup
  const int b = p.b;
  const int rows = p.H_kv * b;
  for (int row0 = 0; row0 < rows; row0 += QT_THREADS) {
    const int row = row0 + (int)threadIdx.x;
    const bool live = row < rows;
    const int h = live ? row / b : 0, t = live ? row % b : 0;
    const size_t head = (size_t)pg * p.H_kv + h;
    if (live) {
      // ---- key row: contiguous, 8 elements per 16-byte load
      const uint16_t* kr = p.k + (head * b + t) * D;
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(kr + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          amax = fmaxf(amax, fmaxf(fabsf(gp::bf16_bits_to_f32(w[e] & 0xffffu)),
                                   fabsf(gp::bf16_bits_to_f32(w[e] >> 16))));
      }
      const _Float16 sh = row_scale(amax);
      const float s = (float)sh;
      uint8_t* k4r = p.k4 + (head * b + t) * (D / 2);
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(kr + 8 * c);
        uint32_t packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          packed |= code_of(gp::bf16_bits_to_f32(w[e] & 0xffffu), s) << (8 * e);
          packed |= code_of(gp::bf16_bits_to_f32(w[e] >> 16), s) << (8 * e + 4);
        }
        *reinterpret_cast<uint32_t*>(k4r + 4 * c) = packed;
      }
      p.k4_scale[head * b + t] = __builtin_bit_cast(uint16_t, sh);
    }
    // ---- value row of token t: element d sits at v[head][d][t]
    const uint16_t* vr = p.v + head * (size_t)D * b + t;
    float amax = 0.f;
    if (live) {
      for (int d = 0; d < D; ++d) amax = fmaxf(amax, fabsf(gp::bf16_bits_to_f32(vr[(size_t)d * b])));
    }
    const _Float16 sh = row_scale(amax);
    const float s = (float)sh;
    if (live) p.v4_scale[head * b + t] = __builtin_bit_cast(uint16_t, sh);
    // rows are b-aligned and b is even, so a token pair never straddles a head or a pass.
    // Block of tokens 4Q .. 4Q+3: dimension j's two bytes sit at slot (j % 16) * (D / 16) + j / 16,
    // byte (t % 4) / 2 of the slot holds tokens t & ~1 (low nibble) and t | 1 (high nibble).
    uint8_t* v4h = p.v4 + head * (size_t)D * (b / 2) + (size_t)(t / 4) * (2 * D) + (t % 4) / 2;
    for (int d = 0; d < D; ++d) {
      const uint32_t c = live ? code_of(gp::bf16_bits_to_f32(vr[(size_t)d * b]), s) : 0u;
      const uint32_t other = __shfl_xor(c, 1, GP_WAVE);
      const int slot = (d % 16) * (D / 16) + d / 16;
      if (live && (t & 1) == 0) v4h[2 * slot] = (uint8_t)(c | (other << 4));
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) p.page_tag[pg] = GP_TAG_INT4;
}

}  // namespace

extern "C" int gp_quantize_pages_int4(const gp_kv_cache* kv, const int32_t* page_ids, int num_ids,
                                      void* stream) {
  if (!kv || num_ids < 0) return GP_ERR_INVALID;
  if (num_ids == 0) return GP_OK;
  if (!page_ids || !kv->k || !kv->v || !kv->page_tag || !kv->k4 || !kv->v4 || !kv->k4_scale ||
      !kv->v4_scale)
    return GP_ERR_INVALID;
  if (kv->dtype != GP_BF16 || kv->num_pages <= 0 || kv->num_kv_heads <= 0) return GP_ERR_INVALID;
  const int D = kv->head_dim, b = kv->page_size;
  if (D != 64 && D != 128) return GP_ERR_UNSUPPORTED;
  if (b < 16 || b > 256 || b % 16 != 0) return GP_ERR_UNSUPPORTED;
  if ((long)kv->num_pages * kv->num_kv_heads * b * D > (1L << 40)) return GP_ERR_INVALID;
  QuantParams p{};
  p.k = static_cast<const uint16_t*>(kv->k);
  p.v = static_cast<const uint16_t*>(kv->v);
  p.k4 = static_cast<uint8_t*>(kv->k4);
  p.v4 = static_cast<uint8_t*>(kv->v4);
  p.k4_scale = kv->k4_scale;
  p.v4_scale = kv->v4_scale;
  p.page_tag = kv->page_tag;
  p.page_ids = page_ids;
  p.num_ids = num_ids;
  p.num_pages = kv->num_pages;
  p.H_kv = kv->num_kv_heads;
  p.b = b;
  p.D = D;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 64)
    hipLaunchKernelGGL(quantize_pages_kernel<64>, dim3(num_ids), dim3(QT_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(quantize_pages_kernel<128>, dim3(num_ids), dim3(QT_THREADS), 0, s, p);
  return hipGetLastError() == hipSuccess ? GP_OK : GP_ERR_HIP;
}
