// Paged decode attention for gfx950 (PASK Sec. 3.1 attention definition, App. B.5 split-KV
// merge and mixed-precision page reads; GrowPage Sec. 4.2 block tables).
//
// Work decomposition: one workgroup (4 wave64s) per (split of a request's tokens, KV head,
// request). A split is a run of 16-token tiles; wave w takes tiles w, w+4, ... of the split.
// Per tile the G query heads of the KV head are contracted against the key tile on the
// matrix cores (keys as the 16-row operand, heads as the 16-column operand, so the result
// lands with one head per lane column), an online softmax runs on the 4 logits each lane holds,
// and the probability tile - already in the operand layout of the next product - is multiplied
// with the value tile (values are stored token-contiguous inside a page, so each lane reads 4
// consecutive tokens of one value row). The four waves merge their (max, sum, output) in LDS;
// with more than one split per request a second kernel merges split partials with the rule of
// PASK App. B.5.
#include "common.h"

namespace {

constexpr int KIND_F32 = 0;
constexpr int KIND_BF16 = 1;
constexpr int KIND_MIXED = 2;
constexpr int WAVES = 4;
constexpr int THREADS = WAVES * GP_WAVE;
constexpr int MAX_SPLIT_TILES = 256;

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* page_tag;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse;
  float* ws_o;   // [B, H_q, num_splits, D]
  float* ws_ml;  // [B, H_q, num_splits, 2]
  int B, H_q, H_kv, G, page_size, num_pages, max_pages, max_context;
  int split_tiles, num_splits;
  float scale_log2;
};

// Raw operand registers of one 16-token tile, as loaded from HBM.
template <int D, int KIND>
struct TileRaw;

template <int D>
struct TileRaw<D, KIND_F32> {
  u32x4_t k[D / 16];  // D/4 key floats of token (lane % 16)
  u32x4_t v[D / 16];  // per 16-row block of values: 4 consecutive tokens of one value row
};

template <int D>
struct TileRaw<D, KIND_BF16> {
  u32x4_t k[D / 32];  // 8 bf16 of the key row per 32-wide k step
  u32x2_t v[D / 16];  // 4 bf16 tokens of one value row per 16-row block
};

template <int D>
struct TileRaw<D, KIND_MIXED> {
  u32x4_t k[D / 32];  // bf16: 8 elements; fp8: 8 codes in .xy
  u32x2_t v[D / 16];  // bf16: 4 elements; fp8: 4 codes in .x
  f32x4_t ks, vs;     // per-token scales of the 4 tokens this lane owns (fp8 pages)
};

__device__ __forceinline__ int sanitize_ctx(const DecodeParams& p, int r) {
  int ctx = p.context_lens[r];
  const long cap = (long)p.max_pages * p.page_size;
  if (ctx < 0 || ctx > p.max_context || ctx > cap) ctx = 0;
  return ctx;
}

template <int D, int KIND>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int code, int tok0, int h,
                                          int lane, TileRaw<D, KIND>& t) {
  const int n16 = lane & 15, g4 = lane >> 4;
  const int b = p.page_size;
  const int off = tok0 % b;
  if constexpr (KIND == KIND_MIXED) {
    const int pg = code >> 2, tag = code & 3;
    const size_t kv_base = ((size_t)pg * p.H_kv + h) * (size_t)b * D;
    if (tag == GP_TAG_FP8) {
      const uint8_t* kr = p.k8 + kv_base + (size_t)(off + n16) * D + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        u32x2_t c = *reinterpret_cast<const u32x2_t*>(kr + 32 * kk);
        t.k[kk] = u32x4_t{c.x, c.y, 0u, 0u};
      }
      const uint8_t* vr = p.v8 + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
        t.v[nb] = u32x2_t{*reinterpret_cast<const uint32_t*>(vr + (size_t)16 * nb * b), 0u};
      const size_t sb = ((size_t)pg * p.H_kv + h) * b + off + 4 * g4;
      t.ks = *reinterpret_cast<const f32x4_t*>(p.k_scale + sb);
      t.vs = *reinterpret_cast<const f32x4_t*>(p.v_scale + sb);
      return;
    }
    const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.k) + kv_base + (size_t)(off + n16) * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = *reinterpret_cast<const u32x4_t*>(kr + 32 * kk);
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.v) + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = *reinterpret_cast<const u32x2_t*>(vr + (size_t)16 * nb * b);
    t.ks = f32x4_t{1.f, 1.f, 1.f, 1.f};
    t.vs = t.ks;
  } else {
    const int pg = code;
    const size_t kv_base = ((size_t)pg * p.H_kv + h) * (size_t)b * D;
    if constexpr (KIND == KIND_BF16) {
      const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.k) + kv_base + (size_t)(off + n16) * D + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = *reinterpret_cast<const u32x4_t*>(kr + 32 * kk);
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.v) + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = *reinterpret_cast<const u32x2_t*>(vr + (size_t)16 * nb * b);
    } else {
      const float* kr = reinterpret_cast<const float*>(p.k) + kv_base + (size_t)(off + n16) * D + (D / 4) * g4;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) t.k[i] = *reinterpret_cast<const u32x4_t*>(kr + 4 * i);
      const float* vr = reinterpret_cast<const float*>(p.v) + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = *reinterpret_cast<const u32x4_t*>(vr + (size_t)16 * nb * b);
    }
  }
}

template <int D, int KIND>
__global__ __launch_bounds__(THREADS) void decode_split_kernel(DecodeParams p) {
  const int s = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int G = p.G;
  const int ctx = sanitize_ctx(p, r);
  const int ntiles = (ctx + 15) >> 4;
  const int t0 = s * p.split_tiles;
  if (s > 0 && t0 >= ntiles) return;
  const int t1 = min(ntiles, t0 + p.split_tiles);

  __shared__ int s_code[MAX_SPLIT_TILES];
  extern __shared__ float s_dyn[];  // m [WAVES][16], l [WAVES][16], o [WAVES][G][D]
  for (int i = threadIdx.x; i < t1 - t0; i += THREADS) {
    const int tok = (t0 + i) << 4;
    int pg = p.block_tables[(size_t)r * p.max_pages + tok / p.page_size];
    int code = (pg >= 0 && pg < p.num_pages) ? pg : -1;
    if constexpr (KIND == KIND_MIXED) {
      if (code >= 0) {
        const int tag = p.page_tag[pg];
        code = (tag == GP_TAG_FP8 || tag == GP_TAG_BF16) ? ((pg << 2) | tag) : -1;
      }
    }
    s_code[i] = code;
  }
  __syncthreads();

  // query operand: head (lane % 16) of this KV head's group, zero rows past G
  const int hq0 = h * G;
  constexpr int NQ = (KIND == KIND_F32) ? D / 4 : D / 32;
  u32x4_t qf[KIND == KIND_F32 ? D / 16 : D / 32];
  if constexpr (KIND == KIND_F32) {
    const float* qr = reinterpret_cast<const float*>(p.q) + ((size_t)r * p.H_q + hq0 + n16) * D + (D / 4) * g4;
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      qf[i] = (n16 < G) ? *reinterpret_cast<const u32x4_t*>(qr + 4 * i) : u32x4_t{0u, 0u, 0u, 0u};
  } else {
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)r * p.H_q + hq0 + n16) * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qf[kk] = (n16 < G) ? *reinterpret_cast<const u32x4_t*>(qr + 32 * kk) : u32x4_t{0u, 0u, 0u, 0u};
  }
  (void)NQ;

  f32x4_t acc[D / 16];
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // running max (log2 domain) of head n16
  float l_run = 0.f;        // this lane's share of the running sum of head n16

  TileRaw<D, KIND> cur, nxt;
  int ti = t0 + w;
  int code_cur = (ti < t1) ? s_code[ti - t0] : -1;
  if (code_cur >= 0) load_tile<D, KIND>(p, code_cur, ti << 4, h, lane, cur);

  for (; ti < t1; ti += WAVES) {
    const int tn = ti + WAVES;
    const int code_nxt = (tn < t1) ? s_code[tn - t0] : -1;
    if (code_nxt >= 0) load_tile<D, KIND>(p, code_nxt, tn << 4, h, lane, nxt);

    if (code_cur >= 0) {
      const int tok0 = ti << 4;
      const bool tail = tok0 + 16 > ctx;
      // ---- logits: S[token 4*g4 + i][head n16]
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
      bool fp8 = false;
      if constexpr (KIND == KIND_MIXED) fp8 = (code_cur & 3) == GP_TAG_FP8;
      if constexpr (KIND == KIND_F32) {
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sacc = gp::mfma_f32_16x16x4(__uint_as_float(cur.k[i][c]), __uint_as_float(qf[i][c]), sacc);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          u32x4_t kw = cur.k[kk];
          if constexpr (KIND == KIND_MIXED) {
            if (fp8) {
              u32x2_t lo = gp::fp8x4_to_bf16x4(kw.x), hi = gp::fp8x4_to_bf16x4(kw.y);
              kw = u32x4_t{lo.x, lo.y, hi.x, hi.y};
            }
          }
          sacc = gp::mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, kw),
                                        __builtin_bit_cast(bf16x8_t, qf[kk]), sacc);
        }
      }
      float sv[4];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float z = sacc[i];
        if constexpr (KIND == KIND_MIXED) z *= cur.ks[i];
        const bool ok = tok0 + 4 * g4 + i < ctx;
        sv[i] = ok ? z * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, sv[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, GP_WAVE));
      mx = fmaxf(mx, __shfl_xor(mx, 32, GP_WAVE));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = gp::safe_exp2_diff(m_run, m_new);
      float pv[4];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = gp::safe_exp2_diff(sv[i], m_new);
        psum += pv[i];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // rescale the output rows: this lane holds heads 4*g4 + i
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g4 + i, GP_WAVE);
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] *= al[i];
      // token validity of the 4 tokens this lane feeds into the value product
      if constexpr (KIND == KIND_F32) {
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          u32x4_t vw = cur.v[nb];
          if (tail) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (tok0 + 4 * g4 + i >= ctx) vw[i] = 0u;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[nb] = gp::mfma_f32_16x16x4(pv[i], __uint_as_float(vw[i]), acc[nb]);
        }
      } else {
        float pw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pw[i] = pv[i];
          if constexpr (KIND == KIND_MIXED) pw[i] *= cur.vs[i];
        }
        if constexpr (KIND == KIND_MIXED) {
          // released or poisoned scales only occur on masked tokens; keep them out of the product
#pragma unroll
          for (int i = 0; i < 4; ++i) if (pv[i] == 0.f) pw[i] = 0.f;
        }
        const u32x2_t pp = u32x2_t{gp::pack_bf16x2(pw[0], pw[1]), gp::pack_bf16x2(pw[2], pw[3])};
        uint32_t mlo = 0xffffffffu, mhi = 0xffffffffu;
        if (tail) {
          const int base = tok0 + 4 * g4;
          mlo = (base + 0 < ctx ? 0x0000ffffu : 0u) | (base + 1 < ctx ? 0xffff0000u : 0u);
          mhi = (base + 2 < ctx ? 0x0000ffffu : 0u) | (base + 3 < ctx ? 0xffff0000u : 0u);
        }
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          u32x2_t vw = cur.v[nb];
          if constexpr (KIND == KIND_MIXED) {
            if (fp8) vw = gp::fp8x4_to_bf16x4(vw.x);
          }
          vw.x &= mlo;
          vw.y &= mhi;
          acc[nb] = gp::mfma_bf16_16x16x16(__builtin_bit_cast(i16x4_t, pp),
                                           __builtin_bit_cast(i16x4_t, vw), acc[nb]);
        }
      }
    }
    cur = nxt;
    code_cur = code_nxt;
  }

  // ---- merge the 4 waves
  float l_tot = l_run + __shfl_xor(l_run, 16, GP_WAVE);
  l_tot += __shfl_xor(l_tot, 32, GP_WAVE);
  float* s_m = s_dyn;
  float* s_l = s_dyn + WAVES * 16;
  float* s_o = s_dyn + 2 * WAVES * 16;
  if (lane < 16) {
    s_m[w * 16 + lane] = m_run;
    s_l[w * 16 + lane] = l_tot;
  }
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 4 * g4 + i;
      if (head < G) s_o[((size_t)w * G + head) * D + 16 * nb + n16] = acc[nb][i];
    }
  __syncthreads();

  const bool final_out = p.num_splits == 1;
  for (int idx = threadIdx.x; idx < G * D; idx += THREADS) {
    const int head = idx / D, dd = idx % D;
    float m = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) m = fmaxf(m, s_m[ww * 16 + head]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) {
      const float e = gp::safe_exp2_diff(s_m[ww * 16 + head], m);
      num += e * s_o[((size_t)ww * G + head) * D + dd];
      den += e * s_l[ww * 16 + head];
    }
    const size_t row = (size_t)r * p.H_q + hq0 + head;
    if (final_out) {
      const float o = den > 0.f ? num / den : 0.f;
      if constexpr (KIND == KIND_F32)
        reinterpret_cast<float*>(p.out)[row * D + dd] = o;
      else
        reinterpret_cast<uint16_t*>(p.out)[row * D + dd] = (uint16_t)gp::f32_to_bf16_bits(o);
      if (dd == 0 && p.lse) p.lse[row] = den > 0.f ? (m + __log2f(den)) * GP_LN2 : -INFINITY;
    } else {
      p.ws_o[(row * p.num_splits + s) * D + dd] = num;
      if (dd == 0) {
        p.ws_ml[(row * p.num_splits + s) * 2 + 0] = m;
        p.ws_ml[(row * p.num_splits + s) * 2 + 1] = den;
      }
    }
  }
}

// Merge of split partials (PASK App. B.5): o = sum_j e^{m_j - m} u_j / sum_j e^{m_j - m} l_j.
template <int D, int KIND>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeParams p) {
  const int hq = blockIdx.x, r = blockIdx.y;
  const int ctx = sanitize_ctx(p, r);
  const int ntiles = (ctx + 15) >> 4;
  int ns = (ntiles + p.split_tiles - 1) / p.split_tiles;
  ns = max(1, min(ns, p.num_splits));
  const size_t row = (size_t)r * p.H_q + hq;
  const float* ml = p.ws_ml + row * p.num_splits * 2;
  float m = -INFINITY;
  for (int j = 0; j < ns; ++j) m = fmaxf(m, ml[2 * j]);
  float den = 0.f;
  for (int j = 0; j < ns; ++j) den += gp::safe_exp2_diff(ml[2 * j], m) * ml[2 * j + 1];
  const float inv = den > 0.f ? 1.f / den : 0.f;
  for (int dd = threadIdx.x; dd < D; dd += 64) {
    float num = 0.f;
    for (int j = 0; j < ns; ++j)
      num += gp::safe_exp2_diff(ml[2 * j], m) * p.ws_o[(row * p.num_splits + j) * D + dd];
    const float o = num * inv;
    if constexpr (KIND == KIND_F32)
      reinterpret_cast<float*>(p.out)[row * D + dd] = o;
    else
      reinterpret_cast<uint16_t*>(p.out)[row * D + dd] = (uint16_t)gp::f32_to_bf16_bits(o);
  }
  if (threadIdx.x == 0 && p.lse) p.lse[row] = den > 0.f ? (m + __log2f(den)) * GP_LN2 : -INFINITY;
}

struct SplitPlan {
  int split_tiles;
  int num_splits;
};

SplitPlan plan_splits(int B, int H_kv, int max_context) {
  const long max_tiles = (max_context + 15) / 16;
  int st = 64;
  while (st > 4 && (long)B * H_kv * ((max_tiles + st - 1) / st) < 4096) st >>= 1;
  SplitPlan sp;
  sp.split_tiles = st;
  sp.num_splits = (int)std::max<long>(1, (max_tiles + st - 1) / st);
  return sp;
}

template <int D, int KIND>
int launch_decode(const DecodeParams& p, hipStream_t stream) {
  dim3 grid(p.num_splits, p.H_kv, p.B);
  const size_t lds = (size_t)(2 * WAVES * 16 + WAVES * p.G * D) * sizeof(float);
  hipLaunchKernelGGL((decode_split_kernel<D, KIND>), grid, dim3(THREADS), lds, stream, p);
  GP_CHECK_LAUNCH();
  if (p.num_splits > 1) {
    hipLaunchKernelGGL((decode_combine_kernel<D, KIND>), dim3(p.H_q, p.B), dim3(64), 0, stream, p);
    GP_CHECK_LAUNCH();
  }
  return GP_OK;
}

}  // namespace

extern "C" size_t gp_paged_decode_attn_workspace_size(int B, int H_q, int H_kv, int head_dim,
                                                      int page_size, int max_context) {
  (void)page_size;
  if (B <= 0 || H_q <= 0 || H_kv <= 0 || head_dim <= 0 || max_context < 0) return 0;
  const SplitPlan sp = plan_splits(B, H_kv, max_context);
  if (sp.num_splits <= 1) return 0;
  return (size_t)B * H_q * sp.num_splits * (head_dim + 2) * sizeof(float);
}

extern "C" int gp_paged_decode_attn(const void* q, int q_dtype, int B, int H_q,
                                    const gp_kv_cache* kv, const int32_t* block_tables,
                                    int max_pages, const int32_t* context_lens, int max_context,
                                    float sm_scale, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (B < 0 || H_q <= 0 || !kv || max_pages <= 0 || max_context < 0) return GP_ERR_INVALID;
  if (B == 0) return GP_OK;
  if (!q || !out || !block_tables || !context_lens || !kv->k || !kv->v) return GP_ERR_INVALID;
  const int H_kv = kv->num_kv_heads, D = kv->head_dim, b = kv->page_size;
  if (H_kv <= 0 || H_q % H_kv != 0 || kv->num_pages <= 0) return GP_ERR_INVALID;
  if (b < 16 || b > 256 || b % 16 != 0) return GP_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return GP_ERR_UNSUPPORTED;
  const int G = H_q / H_kv;
  if (G > 16) return GP_ERR_UNSUPPORTED;
  if (q_dtype != kv->dtype || (q_dtype != GP_F32 && q_dtype != GP_BF16)) return GP_ERR_INVALID;
  const bool mixed = kv->page_tag != nullptr;
  if (mixed && (q_dtype != GP_BF16 || !kv->k8 || !kv->v8 || !kv->k_scale || !kv->v_scale))
    return GP_ERR_INVALID;
  if ((long)max_context > (long)max_pages * b) return GP_ERR_INVALID;
  if ((long)kv->num_pages * H_kv * b > (1L << 40)) return GP_ERR_INVALID;

  const SplitPlan sp = plan_splits(B, H_kv, max_context);
  const size_t need = gp_paged_decode_attn_workspace_size(B, H_q, H_kv, D, b, max_context);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GP_ERR_WORKSPACE;
  if (sp.split_tiles > MAX_SPLIT_TILES) return GP_ERR_INVALID;

  DecodeParams p{};
  p.q = q;
  p.k = kv->k;
  p.v = kv->v;
  p.k8 = static_cast<const uint8_t*>(kv->k8);
  p.v8 = static_cast<const uint8_t*>(kv->v8);
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  p.page_tag = kv->page_tag;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  p.lse = lse;
  p.B = B;
  p.H_q = H_q;
  p.H_kv = H_kv;
  p.G = G;
  p.page_size = b;
  p.num_pages = kv->num_pages;
  p.max_pages = max_pages;
  p.max_context = max_context;
  p.split_tiles = sp.split_tiles;
  p.num_splits = sp.num_splits;
  p.scale_log2 = sm_scale * GP_LOG2E;
  if (sp.num_splits > 1) {
    p.ws_o = static_cast<float*>(workspace);
    p.ws_ml = p.ws_o + (size_t)B * H_q * sp.num_splits * D;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mixed) return D == 64 ? launch_decode<64, KIND_MIXED>(p, s) : launch_decode<128, KIND_MIXED>(p, s);
  if (q_dtype == GP_BF16) return D == 64 ? launch_decode<64, KIND_BF16>(p, s) : launch_decode<128, KIND_BF16>(p, s);
  return D == 64 ? launch_decode<64, KIND_F32>(p, s) : launch_decode<128, KIND_F32>(p, s);
}
