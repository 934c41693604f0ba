// Page-boundary demand estimation for gfx950 (GrowPage App. E.1: Eq. 12 calibration and RoPE of
// the short/long summaries, candidate set without the most recent block, per-view attention with
// the native GQA mapping; Sec. 3.2 Eq. 7 p-coverage working sets). Mixed-precision caches
// (PASK App. B.2 / B.5 pages): fp8 and INT4 keys enter as their exact code values with the row
// scale applied to the dot product, and released tokens are left out of every softmax.
//
// Two launches:
//   1. logits:    each workgroup first RMS-calibrates the 2G summaries of its KV head to q_t and
//                 rotates them to the current position (float64 arithmetic, into LDS), then
//                 contracts its chunk of candidate key tiles with them on the matrix cores
//                 (keys as the 16-row operand, the 2G summaries as columns; bf16 keys meet a
//                 hi+lo bf16 split of the fp32 summaries, fp32 keys use the fp32 MFMA); logits
//                 go to the workspace with per-chunk (max, sum).
//   2. working set: per (request, KV head, view) first the weights: the softmax of each of the
//                 G query heads' rows and their mean, written to a^S / a^L and kept in
//                 registers; then the p-coverage size, exact on those fp32 weights: a binary
//                 search over the weight bit patterns (float32 sums per thread, float64 across
//                 threads) finds the threshold weight, which an exact 160-bit fixed-point sum
//                 then certifies (and corrects if rounding picked a neighbour). Normalising in
//                 the same kernel saves a launch and a write-then-read of the weights, which
//                 matters most when the pass runs beside a decode that keeps HBM busy.
#include "common.h"

#include <algorithm>
#include <cmath>

namespace {

// Waves per logits workgroup: eight when the call has few workgroups (a wave's tiles and
// calibration rows are then fewer, so each workgroup finishes sooner), four otherwise (less
// per-workgroup setup for the same bytes). The kernel reads its count from blockDim.
constexpr int LG_MAX_WAVES = 8;
constexpr int LG_MIN_WAVES = 4;
constexpr long LG_FEW_WORKGROUPS = 1024;
constexpr int CAL_ROWS = (16 + LG_MIN_WAVES - 1) / LG_MIN_WAVES;  // calibrated rows per wave (2G <= 16)
constexpr int LG_MAX_THREADS = LG_MAX_WAVES * GP_WAVE;
constexpr int CHUNK_TILES = 32;  // 512 candidate tokens per logits workgroup
constexpr int WS_THREADS = 1024;
constexpr int WS_VPT = 32;        // weights per thread held in registers (|C| <= 32768)
constexpr int WS_MAX_C = WS_THREADS * WS_VPT;
constexpr int WS_TAIL = 64;       // weights left in the search interval when one wave sorts them
constexpr int WS_TK = WS_TAIL / 64;  // tail keys per lane
// First level of the threshold search: 4096 bins of a weight's bit pattern >> 18 (sign, exponent
// and five mantissa bits: a weight <= 1 has a pattern below 2^30), each holding the bin's count
// (bits 48..63) and mass in units of 2^-47 (bits 0..47: a distribution's total stays below 2).
constexpr int WS_BIN_SHIFT = 18;
constexpr int WS_BINS = 4096;
constexpr int WS_MASS_BITS = 47;
// Relative rounding bound of a block's float64 sum of nonnegative weights: a thread adds its (at
// most 32) weights in sequence, a wave reduces in 6 levels, the 16 wave partials in 4: at most 42
// roundings on any path, each a relative 2^-53; the bound takes 64.
constexpr double SUM_ERR = 64.0 * 0x1p-53;

struct ScoreParams {
  const void* q;
  const float* qstate;
  const int32_t* slot_ids;
  const int32_t* req_idx;
  const void* k;
  const uint8_t* page_tag;  // mixed-precision cache: per-page tag, else null
  const uint8_t* k8;        // fp8 key codes [pages, H_kv, b, D]
  const float* k_scale;     // fp8 row scales [pages, H_kv, b]
  const uint8_t* k4;        // INT4 key codes [pages, H_kv, b, D/2]
  const uint16_t* k4_scale; // INT4 row scales, half bits [pages, H_kv, b]
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* positions;
  float* a_short;
  float* a_long;
  int32_t* ws_counts;
  int32_t* n_cand;
  float* logits;  // [R, 2, H_q, C_max]  (log2 domain)
  float* stats;   // [R, 2, H_q, NCH, 2]
  int B, R, H_q, H_kv, G, D, page_size, num_pages, max_pages, num_slots, C_max, nch;
  int q_bf16;
  float scale_log2;
  double rope_theta;
  double inv_freq[64];  // rope_theta^(-2j/D), j < D/2 (float64, from the host)
  uint32_t p_fixed[5];  // p in units of 2^-149, little-endian 32-bit digits (rounded up)
};

// |C| of request r from its state slot and length (or -1 for an invalid request / slot, or
// |C| > C_max)
__device__ __forceinline__ int candidates_of(const ScoreParams& P, int r, int slot, int ctx) {
  if (r < 0 || r >= P.B) return -1;
  if (slot < 0 || slot >= P.num_slots) return -1;
  if (ctx < 0 || (long)ctx > (long)P.max_pages * P.page_size) return -1;
  if (ctx == 0) return 0;
  const int used = (ctx + P.page_size - 1) / P.page_size;
  const int n = (used - 1) * P.page_size;
  return n > P.C_max ? -1 : n;
}


// ------------------------------------------------------------------------------ 1. calibration
// The 2G summary rows of KV head h of boundary request i (row c = view c / G, query head
// h G + c % G), RMS-calibrated to q_t (Eq. 12) and rotated to the current position, in float64,
// into s_qt[c][0 .. D). One wave per row (a wave takes rows w, w + waves, ...).
__device__ __forceinline__ void calibrated_rows(const ScoreParams& P, int i, int r, int h,
                                                int slot, double pos, double inv_freq, float (*s_qt)[128]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  const int D = P.D, half = D / 2, G = P.G;
  // this wave's rows (at most CAL_ROWS of the 2G <= 16): every query and summary element they
  // need is loaded before any is used
  // (one load form for both query dtypes, the 32-bit word holding the element: a dtype select
  // per element made the compiler branch per load and wait for each load before the next)
  double qv[CAL_ROWS][2], sv[CAL_ROWS][2];
  const bool qb = P.q_bf16 != 0;
  const int qsh = qb ? 1 : 2;  // log2 of the query element size
  const uint8_t* q8 = static_cast<const uint8_t*>(P.q);
#pragma unroll
  for (int k = 0; k < CAL_ROWS; ++k) {
    const int c = w + k * nwv;
    const int cc = c < 2 * G ? c : 0;  // rows past 2G read row 0, unused
    const int x = cc / G, g = h * G + cc % G;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = min(lane + 64 * e, D - 1);
      const size_t qbyte = (((size_t)r * P.H_q + g) * D + d) << qsh;
      const uint32_t wq = *reinterpret_cast<const uint32_t*>(q8 + (qbyte & ~(size_t)3)) >> (8 * (qbyte & 3));
      qv[k][e] = (double)(qb ? gp::bf16_bits_to_f32(wq & 0xffffu) : __uint_as_float(wq));
      sv[k][e] = (double)P.qstate[(((size_t)slot * 2 + x) * P.H_q + g) * D + d];
    }
  }
  // the rotation angle depends on the pair index only: lane l holds elements l and l + 64, and
  // both belong to pair l % (D/2), so one sine and cosine per lane serve every row
  double sn = 0.0, cs = 1.0;
  if (P.rope_theta > 0.0) sincos(pos * inv_freq, &sn, &cs);
#pragma unroll
  for (int k = 0; k < CAL_ROWS; ++k) {
    const int c = w + k * nwv;
    if (c >= 2 * G) continue;  // uniform over the wave
    double sq = 0.0, ss = 0.0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      if (lane + 64 * e < D) {
        sq += qv[k][e] * qv[k][e];
        ss += sv[k][e] * sv[k][e];
      }
    }
    sq = gp::wave_sum_f64(sq);
    ss = gp::wave_sum_f64(ss);
    const double gamma = ss > 0.0 ? sqrt(sq / ss) : 0.0;  // RMS ratio (the 1/D cancels)
    const double cv[2] = {gamma * sv[k][0], gamma * sv[k][1]};
    // the partner of element d is d +/- D/2: lane-local when D == 128, a shuffle when 64
    double part[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) part[e] = D == 128 ? cv[1 - e] : __shfl_xor(cv[0], 32, GP_WAVE);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d >= D) continue;
      double out = cv[e];
      if (P.rope_theta > 0.0)  // d % half == lane % half
        out = (d < half) ? cv[e] * cs - part[e] * sn : part[e] * sn + cv[e] * cs;
      s_qt[c][d] = (float)out;
    }
  }
}

// ------------------------------------------------------------------------------ 2. logits
template <int D, bool BF16, bool MIXED>
__global__ __launch_bounds__(LG_MAX_THREADS) void logits_kernel(ScoreParams P) {
  // heads vary fastest over the grid, so the KV heads of a page (adjacent in HBM) are read by
  // neighbouring workgroups at the same time
  const int h = blockIdx.x, chunk = blockIdx.y, i = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nwv = blockDim.x >> 6;
  const int tile0 = chunk * CHUNK_TILES;
  // Once the request index is known, every load that depends only on it goes out together: the
  // state slot and length (which decide |C|), the position, this lane's rotation frequency and
  // the page id of this lane's tile of the chunk (read before |C| is known, at an index kept
  // inside the request's block-table row, and dropped below when past |C|)
  const int r = gp::uni(P.req_idx[i]);
  if (P.B <= 0) {  // no request is valid (and no row may be read)
    if (h == 0 && chunk == 0 && threadIdx.x == 0) P.n_cand[i] = -1;
    return;
  }
  const int rc = min(max(r, 0), P.B - 1);
  const int slot = P.slot_ids[rc];
  const int ctx = P.context_lens[rc];
  const double pos = (double)P.positions[rc];
  const double inv_freq = P.inv_freq[lane % (D / 2)];
  const int pg_raw = P.block_tables[(size_t)rc * P.max_pages +
                                    min(((tile0 + w + lane * nwv) << 4) / P.page_size, P.max_pages - 1)];
  const int n = gp::uni(candidates_of(P, r, slot, ctx));
  if (h == 0 && chunk == 0 && threadIdx.x == 0) P.n_cand[i] = n;
  if (n <= 0 || tile0 * 16 >= n) return;
  const int tile1 = min(n >> 4, tile0 + CHUNK_TILES);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int G = P.G, b = P.page_size;
  const bool col_ok = n16 < 2 * G;
  const int x = n16 / G, g = n16 % G;
  const int hq = h * G + g;
  // this wave's tiles are tile0 + w + k nwv, k < nt (nt <= CHUNK_TILES / nwv): lane k
  // fetches the page id and tag of tile k up front, and the key rows of plain (bf16 / fp32)
  // tiles are loaded two tiles ahead of their use, with no branch around the loads (a tile
  // past the wave's last, or of another format, reads the pool's first bytes and is unused)
  constexpr int NKW = BF16 ? D / 32 : D / 16;  // 16-byte key pieces of a plain tile per lane
  const int nt = tile1 > tile0 + w ? (tile1 - tile0 - w + nwv - 1) / nwv : 0;
  int pg_l = -1, tag_l = GP_TAG_BF16;
  if (lane < nt) {
    const int pg = pg_raw;
    bool ok = pg >= 0 && pg < P.num_pages;
    if (ok && P.page_tag) {
      tag_l = P.page_tag[pg];
      ok = tag_l != GP_TAG_RELEASE;  // released tokens take no part in the softmax
    }
    pg_l = ok ? pg : -1;
  }
  auto load_plain = [&](int k, u32x4_t (&kw)[NKW]) {
    const int kc = min(k, 63);
    const int pg = __builtin_amdgcn_readlane(pg_l, kc), tag = __builtin_amdgcn_readlane(tag_l, kc);
    const int tok0 = (tile0 + w + k * nwv) << 4;
    const bool plain = k < nt && pg >= 0 && tag == GP_TAG_BF16;
    const size_t base = plain ? ((size_t)pg * P.H_kv + h) * (size_t)b * D + (size_t)(tok0 % b + n16) * D : 0;
    if constexpr (BF16) {
      const u32x4_t* kr = reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(P.k) + base + (plain ? 8 * g4 : 0));
#pragma unroll
      for (int kk = 0; kk < NKW; ++kk) kw[kk] = kr[plain ? 4 * kk : 0];
    } else {
      const u32x4_t* kr = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(P.k) + base + (plain ? (D / 4) * g4 : 0));
#pragma unroll
      for (int c = 0; c < NKW; ++c) kw[c] = kr[plain ? c : 0];
    }
  };
  // the first two tiles' keys are in flight while the summaries are calibrated
  u32x4_t ring[2][NKW];
  load_plain(0, ring[0]);
  load_plain(1, ring[1]);

  // the calibrated, rotated summaries of this KV head (each workgroup of the head computes them:
  // a few hundred float64 operations, cheaper than a launch of their own,
  // and hidden behind the first key loads)
  __shared__ float s_qt[16][128];
  calibrated_rows(P, i, r, h, slot, pos, inv_freq, s_qt);
  __syncthreads();
  // columns past 2G read the first summary row (no branch around the loads) and use zeros
  const float* qrow = s_qt[col_ok ? n16 : 0];

  // summary operand: column n16 = (view x, head g)
  u32x4_t qhi[BF16 ? D / 32 : D / 16], qlo[BF16 ? D / 32 : 1];
  if constexpr (BF16) {
    float2 qv[D / 32][4];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qv[kk][e] = *reinterpret_cast<const float2*>(qrow + 32 * kk + 8 * g4 + 2 * e);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = col_ok ? qv[kk][e].x : 0.f, v1 = col_ok ? qv[kk][e].y : 0.f;
        const uint32_t h0 = gp::f32_to_bf16_bits(v0), h1 = gp::f32_to_bf16_bits(v1);
        hi[e] = h0 | (h1 << 16);
        lo[e] = gp::pack_bf16x2(v0 - gp::bf16_bits_to_f32(h0), v1 - gp::bf16_bits_to_f32(h1));
      }
      qhi[kk] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
      qlo[kk] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(qrow + (D / 4) * g4 + 4 * c);
      qhi[c] = col_ok ? __builtin_bit_cast(u32x4_t, v) : u32x4_t{0u, 0u, 0u, 0u};
    }
    (void)qlo;
  }

  float m_run = -INFINITY, l_run = 0.f;
  float* lrow = P.logits + (((size_t)i * 2 + x) * P.H_q + hq) * P.C_max;
  auto process = [&](int k, const u32x4_t (&kw)[NKW]) {
    const int pg = __builtin_amdgcn_readlane(pg_l, k), tag = __builtin_amdgcn_readlane(tag_l, k);
    const int tok0 = (tile0 + w + k * nwv) << 4;
    const bool valid_page = pg >= 0;
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
    // fp8 / INT4 pages exist only in a mixed cache (its own instantiation: a plain cache's kernel
    // has no load behind this branch, so its waits cover each tile's own loads only)
    if (MIXED && valid_page && tag != GP_TAG_BF16) {
      if constexpr (BF16 && MIXED) {
        // fp8 / INT4 keys: the codes are exact bf16 values; the row scale multiplies the
        // finished dot products (rows 4 g4 + e of the tile)
        const size_t row0 = ((size_t)pg * P.H_kv + h) * (size_t)b + tok0 % b;
        f32x4_t sc;
        if (tag == GP_TAG_FP8) {
          const uint8_t* kr = P.k8 + (row0 + n16) * D + 8 * g4;
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            const u32x2_t c = *reinterpret_cast<const u32x2_t*>(kr + 32 * kk);
            const u32x2_t lo = gp::fp8x4_to_bf16x4(c.x), hi = gp::fp8x4_to_bf16x4(c.y);
            const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
            sacc = gp::mfma_bf16_16x16x32(kb, __builtin_bit_cast(bf16x8_t, qhi[kk]), sacc);
            sacc = gp::mfma_bf16_16x16x32(kb, __builtin_bit_cast(bf16x8_t, qlo[kk]), sacc);
          }
          sc = *reinterpret_cast<const f32x4_t*>(P.k_scale + row0 + 4 * g4);
        } else {
          const uint8_t* kr = P.k4 + (row0 + n16) * (D / 2) + 4 * g4;
#pragma unroll
          for (int kk = 0; kk < D / 32; ++kk) {
            const uint32_t w4 = *reinterpret_cast<const uint32_t*>(kr + 16 * kk);
            uint32_t e2[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c0 = (int32_t)(w4 << (28 - 8 * e)) >> 28;  // nibble 2e
              const int c1 = (int32_t)(w4 << (24 - 8 * e)) >> 28;  // nibble 2e + 1
              e2[e] = (__float_as_uint((float)c0) >> 16) | (__float_as_uint((float)c1) & 0xffff0000u);
            }
            const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, u32x4_t{e2[0], e2[1], e2[2], e2[3]});
            sacc = gp::mfma_bf16_16x16x32(kb, __builtin_bit_cast(bf16x8_t, qhi[kk]), sacc);
            sacc = gp::mfma_bf16_16x16x32(kb, __builtin_bit_cast(bf16x8_t, qlo[kk]), sacc);
          }
          const u32x2_t hs = *reinterpret_cast<const u32x2_t*>(P.k4_scale + row0 + 4 * g4);
          sc = f32x4_t{gp::half_lo(hs.x), gp::half_hi(hs.x), gp::half_lo(hs.y), gp::half_hi(hs.y)};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[e] *= sc[e];
      }
    } else if (valid_page) {
      if constexpr (BF16) {
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          sacc = gp::mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, kw[kk]), __builtin_bit_cast(bf16x8_t, qhi[kk]), sacc);
          sacc = gp::mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, kw[kk]), __builtin_bit_cast(bf16x8_t, qlo[kk]), sacc);
        }
      } else {
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc = gp::mfma_f32_16x16x4(__uint_as_float(kw[c][e]), __uint_as_float(qhi[c][e]), sacc);
        }
      }
    }
    f32x4_t z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = valid_page ? sacc[e] * P.scale_log2 : -INFINITY;
    if (col_ok) *reinterpret_cast<f32x4_t*>(lrow + tok0 + 4 * g4) = z;
    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    const float m_new = fmaxf(m_run, mx);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) s += gp::safe_exp2_diff(z[e], m_new);
    l_run = l_run * gp::safe_exp2_diff(m_run, m_new) + s;
    m_run = m_new;
  };
  for (int k0 = 0; k0 < nt; k0 += 2) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (k0 + q < nt) process(k0 + q, ring[q]);
      load_plain(k0 + q + 2, ring[q]);  // past the wave's last tile: the pool's first bytes, unused
    }
  }
  // merge the 4 lanes of each column, then the waves
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float mo = __shfl_xor(m_run, o, GP_WAVE), lo_ = __shfl_xor(l_run, o, GP_WAVE);
    const float mm = fmaxf(m_run, mo);
    l_run = l_run * gp::safe_exp2_diff(m_run, mm) + lo_ * gp::safe_exp2_diff(mo, mm);
    m_run = mm;
  }
  __shared__ float sm[LG_MAX_WAVES][16], sl[LG_MAX_WAVES][16];
  if (lane < 16) {
    sm[w][lane] = m_run;
    sl[w][lane] = l_run;
  }
  __syncthreads();
  if (threadIdx.x < 2 * G) {
    const int c = threadIdx.x;
    float m = -INFINITY;
    for (int ww = 0; ww < nwv; ++ww) m = fmaxf(m, sm[ww][c]);
    float l = 0.f;
    for (int ww = 0; ww < nwv; ++ww) l += sl[ww][c] * gp::safe_exp2_diff(sm[ww][c], m);
    const int xx = c / G, gg = c % G;
    float* st = P.stats + ((((size_t)i * 2 + xx) * P.H_q + h * G + gg) * P.nch + chunk) * 2;
    st[0] = m;
    st[1] = l;
  }
}

// ------------------------------------------------------------------------------ 3. working set
// 160-bit fixed point in units of 2^-149, accumulated as five 32-bit digits held in 64-bit
// counters (carries are resolved once, after the block reduction).
struct Acc5 {
  uint64_t d[6];
};

__device__ __forceinline__ void acc_add(Acc5& a, uint32_t bits) {
  const uint32_t E = bits >> 23;
  if (bits == 0u) return;
  uint32_t M = bits & 0x7fffffu;
  uint32_t sh = 0;
  if (E) {
    M |= 0x800000u;
    sh = min(E, 129u) - 1u;
  }
  const uint64_t v = (uint64_t)M << (sh & 31u);
  const uint32_t k0 = sh >> 5;
  const uint64_t lo = v & 0xffffffffull, hi = v >> 32;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    a.d[k] += (k == (int)k0) ? lo : 0ull;
    a.d[k] += (k == (int)k0 + 1) ? hi : 0ull;
  }
}

// a += count * value(bits), exact (count * mantissa < 2^40)
__device__ __forceinline__ void acc_add_mul(Acc5& a, uint32_t bits, uint32_t count) {
  const uint32_t E = bits >> 23;
  if (bits == 0u || count == 0u) return;
  uint32_t M = bits & 0x7fffffu;
  uint32_t sh = 0;
  if (E) {
    M |= 0x800000u;
    sh = min(E, 129u) - 1u;
  }
  const unsigned __int128 v = (unsigned __int128)((uint64_t)M * count) << (sh & 31u);
  const uint32_t k0 = sh >> 5;
  const uint64_t d0 = (uint64_t)v & 0xffffffffull, d1 = (uint64_t)(v >> 32) & 0xffffffffull,
                 d2 = (uint64_t)(v >> 64);
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    a.d[k] += (k == (int)k0) ? d0 : 0ull;
    a.d[k] += (k == (int)k0 + 1) ? d1 : 0ull;
    a.d[k] += (k == (int)k0 + 2) ? d2 : 0ull;
  }
}

// normalise carries into 6 clean 32-bit digits
__device__ __forceinline__ void acc_norm(const Acc5& a, uint32_t out[6]) {
  uint64_t carry = 0;
#pragma unroll
  for (int k = 0; k < 6; ++k) {
    const uint64_t t = a.d[k] + carry;
    out[k] = (uint32_t)t;
    carry = t >> 32;
  }
}

// compare a (6 digits) with p (5 digits): returns -1, 0, 1
__device__ __forceinline__ int cmp_p(const uint32_t a[6], const uint32_t p[5]) {
  if (a[5]) return 1;
  for (int k = 4; k >= 0; --k) {
    if (a[k] != p[k]) return a[k] < p[k] ? -1 : 1;
  }
  return 0;
}

// Bitonic sort, descending, of 64 TK keys held TK per lane by one wave (key k * 64 + lane in
// x[k]): partners 64 or more keys apart sit in this lane's own registers, nearer ones in other
// lanes of the same register.
template <int SIZE, int J, int TK>
__device__ __forceinline__ void bitonic_step(uint32_t (&x)[TK], int lane) {
  if constexpr (J >= GP_WAVE) {
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      if (k & (J / GP_WAVE)) continue;
      const int k2 = k | (J / GP_WAVE);
      const bool desc = ((k * GP_WAVE + lane) & SIZE) == 0;  // the same for k2 (J < SIZE)
      const uint32_t a = x[k], b = x[k2];
      x[k] = desc ? max(a, b) : min(a, b);
      x[k2] = desc ? min(a, b) : max(a, b);
    }
  } else {
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      uint32_t hi, lo;
      gp::lane_pair_minmax<J>(x[k], hi, lo);
      const bool lower = (lane & J) == 0;
      const bool desc = ((k * GP_WAVE + lane) & SIZE) == 0;
      x[k] = lower == desc ? hi : lo;
    }
  }
  if constexpr (J > 1) bitonic_step<SIZE, J / 2, TK>(x, lane);
}
template <int SIZE, int TK>
__device__ __forceinline__ void bitonic_sort_desc(uint32_t (&x)[TK], int lane) {
  if constexpr (SIZE > 2) bitonic_sort_desc<SIZE / 2, TK>(x, lane);
  bitonic_step<SIZE, SIZE / 2, TK>(x, lane);
}
constexpr int WS_WAVES = WS_THREADS / GP_WAVE;
static_assert(WS_WAVES <= 16, "block reductions hand one partial per wave to the 16 lanes of a DPP row");

__global__ __launch_bounds__(WS_THREADS) void working_set_kernel(ScoreParams P) {
  const int row = blockIdx.x, i = blockIdx.y;
  const int h = row >> 1, x = row & 1;
  int32_t* out = P.ws_counts + ((size_t)i * P.H_kv + h) * 2 + x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = P.G;
  // Once the request index is known, the loads that depend only on it go out together: the
  // state slot and length (which decide |C|), the first batch of logits (four per thread and
  // query head, at indices kept inside the row) and each query head's per-chunk (max, sum)
  // pairs (every chunk slot of the row); what lies past |C| is dropped once |C| is known.
  const int r = gp::uni(P.req_idx[i]);
  if (P.B <= 0) {  // no request is valid (and no row may be read)
    if (threadIdx.x == 0) *out = -1;
    return;
  }
  const int rc = min(max(r, 0), P.B - 1);
  const int slot = P.slot_ids[rc];
  const int ctx = P.context_lens[rc];
  const float* lg0 = P.logits + (((size_t)i * 2 + x) * P.H_q + h * G) * P.C_max;
  float z0[8][4];
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min((int)threadIdx.x + j * WS_THREADS, P.C_max - 1);
      z0[g][j] = g < G ? lg0[(size_t)g * P.C_max + t] : 0.f;
    }
  float mj_raw = -INFINITY, lj_raw = 0.f;
  if (w < G && lane < P.nch) {
    const float* st = P.stats + (((size_t)i * 2 + x) * P.H_q + h * G + w) * P.nch * 2;
    mj_raw = st[2 * lane];
    lj_raw = st[2 * lane + 1];
  }
  const int n = gp::uni(candidates_of(P, r, slot, ctx));
  if (n <= 0) {
    if (threadIdx.x == 0) *out = n < 0 ? -1 : 0;
    return;
  }
  constexpr int NT = WS_THREADS;
  // weights per thread that can be candidates: the rest of a thread's 32 slots hold zeros, which
  // no sum, count or maximum below depends on, so the loops skip them (a uniform bound)
  const int nv = (n + NT - 1) / NT;
  // Block reductions with one barrier each: wave partials alternate between two scratch
  // buffers, so a buffer is rewritten only after every thread has passed another barrier.
  __shared__ double s_d[2][WS_WAVES];
  __shared__ uint32_t s_dc[2][WS_WAVES];
  __shared__ uint64_t s_u[2][8][WS_WAVES];
  __shared__ uint32_t s_x[2][WS_WAVES];
  int ph = 0;
  constexpr int BPT = WS_BINS / WS_THREADS;  // histogram bins per thread
  static_assert(BPT * WS_THREADS == WS_BINS, "whole bins per thread");
  __shared__ unsigned long long s_hist[WS_BINS];
  __shared__ int s_bin;
  __shared__ unsigned long long s_bin_incl, s_bin_excl;
  __shared__ unsigned long long s_wtot[WS_WAVES];
#pragma unroll
  for (int k = 0; k < BPT; ++k) s_hist[k * WS_THREADS + threadIdx.x] = 0ull;
  if (threadIdx.x == 0) s_bin = -1;
  // a float64 sum and an integer count in one barrier
  auto sum_dc = [&](double v, uint32_t c, uint32_t* c_out) -> double {
    v = gp::wave_sum_f64(v);
    const uint32_t cw = gp::wave_sum_u32(c);
    if (lane == 0) {
      s_d[ph][w] = v;
      s_dc[ph][w] = cw;
    }
    __syncthreads();
    // lane k of every row takes wave k's partial; the row reduction leaves the total everywhere
    const int k = lane & 15;
    const double t = gp::row16_sum_f64(k < WS_WAVES ? s_d[ph][k] : 0.0);
    const uint32_t tc = gp::row16_sum_u32(k < WS_WAVES ? s_dc[ph][k] : 0u);
    ph ^= 1;
    *c_out = gp::uni(tc);
    return gp::uni(t);
  };
  auto sum_u8 = [&](uint64_t (&v)[8]) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      v[c] = gp::wave_sum_u64(v[c]);
      if (lane == 0) s_u[ph][c][w] = v[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = gp::uni(gp::row16_sum_u64((lane & 15) < WS_WAVES ? s_u[ph][c][lane & 15] : 0ull));
    ph ^= 1;
  };
  // the sum, the count and the maximum in one barrier
  auto sum_cnt_max = [&](double v, uint32_t c, uint32_t m, uint32_t* c_out, uint32_t* m_out) -> double {
    v = gp::wave_sum_f64(v);
    c = gp::wave_sum_u32(c);
    m = gp::wave_max_u32(m);
    if (lane == 0) {
      s_d[ph][w] = v;
      s_dc[ph][w] = c;
      s_x[ph][w] = m;
    }
    __syncthreads();
    const int k = lane & 15;
    const double t = gp::row16_sum_f64(k < WS_WAVES ? s_d[ph][k] : 0.0);
    const uint32_t tc = gp::row16_sum_u32(k < WS_WAVES ? s_dc[ph][k] : 0u);
    const uint32_t tm = gp::row16_max_u32(k < WS_WAVES ? s_x[ph][k] : 0u);
    ph ^= 1;
    *c_out = gp::uni(tc);
    *m_out = gp::uni(tm);
    return gp::uni(t);
  };
  auto max_x = [&](uint32_t v) -> uint32_t {
    v = gp::wave_max_u32(v);
    if (lane == 0) s_x[ph][w] = v;
    __syncthreads();
    const uint32_t t = gp::row16_max_u32((lane & 15) < WS_WAVES ? s_x[ph][lane & 15] : 0u);
    ph ^= 1;
    return gp::uni(t);
  };

  // ---- this row's weights (GrowPage Sec. 3.2): the softmax over C of each of the G query heads
  // of KV head h in view x, from the logits and the per-chunk (max, sum) pairs the logits
  // kernel left, then their mean; written to a^x and kept in registers for the search
  // later batches: indexes past the candidates read candidate 0 (no branch per element) and are
  // dropped below
  auto load_batch = [&](int j0, float (&z)[8][4]) {
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = threadIdx.x + (j0 + j) * NT;
        z[g][j] = (g < G && j0 + j < nv) ? lg0[(size_t)g * P.C_max + (t < n ? t : 0)] : 0.f;
      }
  };
  __shared__ float s_m[16], s_inv[16];
  {
    // one wave per query head: lane j holds chunk j's (max, sum)
    const int nchunks = (n + CHUNK_TILES * 16 - 1) / (CHUNK_TILES * 16);  // <= 64
    static_assert(WS_WAVES >= 8, "one wave per query head (G <= 8)");
    if (w < G) {
      const int g = w;
      const float mj = lane < nchunks ? mj_raw : -INFINITY;
      const float lj = lane < nchunks ? lj_raw : 0.f;
      const float m = gp::wave_max(mj);
      const float l = gp::wave_sum(lj * gp::safe_exp2_diff(mj, m));
      if (lane == 0) {
        s_m[g] = m;
        s_inv[g] = l > 0.f ? 1.f / l : 0.f;
      }
    }
    __syncthreads();
  }
  float* dst = (x == 0 ? P.a_short : P.a_long) + ((size_t)i * P.H_kv + h) * P.C_max;
  uint32_t u[WS_VPT];
  {
    float acc[WS_VPT];
#pragma unroll
    for (int j = 0; j < WS_VPT; ++j) acc[j] = 0.f;
    // four weights of every query head per batch, all loads of a batch issued before any is used
#pragma unroll
    for (int j0 = 0; j0 < WS_VPT; j0 += 4) {
      if (j0 >= nv) continue;  // uniform: skips the batch without breaking the unrolling
      float z[8][4];
      if (j0 == 0) {
#pragma unroll
        for (int g = 0; g < 8; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j) z[g][j] = z0[g][j];
      } else {
        load_batch(j0, z);
      }
#pragma unroll
      for (int g = 0; g < 8; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (g < G && j0 + j < nv) acc[j0 + j] += gp::safe_exp2_diff(z[g][j], s_m[g]) * s_inv[g];
    }
    const float invG = 1.0f / (float)G;
#pragma unroll
    for (int j = 0; j < WS_VPT; ++j) {
      const int t = threadIdx.x + j * NT;
      const float v = acc[j] * invG;
      const bool mine = j < nv && t < n;
      if (mine) dst[t] = v;
      u[j] = mine ? __float_as_uint(v) & 0x7fffffffu : 0u;
    }
  }
  // the loops below take a thread's weights u[0 .. nv) in groups of four, with one uniform test
  // per group: the slots past nv hold 0, which no loop counts, sums or takes as a maximum
  auto each = [&](auto&& f) {
#pragma unroll
    for (int j0 = 0; j0 < WS_VPT; j0 += 4) {
      if (j0 < nv) {
#pragma unroll
        for (int j = j0; j < j0 + 4; ++j) f(j);
      }
    }
  };
  double p_f64 = 0.0;
  for (int k = 4; k >= 0; --k) p_f64 = p_f64 * 4294967296.0 + (double)P.p_fixed[k];
  p_f64 = ldexp(p_f64, -149);

  // Total mass: if it never reaches p, K = |C|; also the largest weight and the count of nonzero
  // weights. The float64 sum of the nonnegative weights is within SUM_ERR of the exact one
  // (relative), so it decides unless p lies inside that bound; then the exact 160-bit sum does.
  uint32_t vmax, n_nz;
  {
    double ts = 0.0;
    uint32_t m = 0u, c = 0u;
    each([&](int j) {
      ts += (double)__uint_as_float(u[j]);
      m = max(m, u[j]);
      c += u[j] != 0u;
      // the weight's bin: one count and its mass in units of 2^-47 (truncated)
      if (u[j] != 0u) {
        const uint32_t E = u[j] >> 23;
        const uint64_t M = E ? ((u[j] & 0x7fffffu) | 0x800000u) : (u[j] & 0x7fffffu);
        const int sh = (E ? (int)E : 1) - 150 + WS_MASS_BITS;  // value = M * 2^(sh - 47)
        const uint64_t fx = sh >= 0 ? (M << sh) : (-sh < 64 ? (M >> -sh) : 0ull);
        atomicAdd(&s_hist[min(u[j] >> WS_BIN_SHIFT, (uint32_t)WS_BINS - 1u)], (1ull << 48) | fx);
      }
    });
    const double tot_f = sum_cnt_max(ts, c, m, &n_nz, &vmax);
    const double err = SUM_ERR * tot_f;
    bool below = tot_f + err < p_f64;
    if (!below && tot_f - err < p_f64) {  // undecided: exact
      Acc5 a = {};
#pragma unroll
      for (int j = 0; j < WS_VPT; ++j)
        if (j < nv) acc_add(a, u[j]);
      uint64_t t[8] = {a.d[0], a.d[1], a.d[2], a.d[3], a.d[4], a.d[5], 0ull, 0ull};
      sum_u8(t);
      Acc5 tt;
#pragma unroll
      for (int k = 0; k < 6; ++k) tt.d[k] = t[k];
      uint32_t tot[6];
      acc_norm(tt, tot);
      below = cmp_p(tot, P.p_fixed) < 0;
    }
    if (below) {
      if (threadIdx.x == 0) *out = n;
      return;
    }
  }
  // search for the largest bit pattern T with mass(weights >= T) >= p: first the histogram bin
  // that holds it (counts and fixed-point masses gathered while the total was summed), then
  // bisection inside the bin. A thread's 32 weights are summed in float32 (the search only has to
  // land on or next to the threshold; the certificate below decides exactly), threads in float64.
  // Each block-wide step also counts the weights at or above its midpoint; once at most WS_TAIL
  // weights lie in [lo, hi), they are listed in LDS and one wave finishes the search without
  // barriers: it sorts them and walks a running sum down from the mass at or above hi.
  uint32_t lo = 1u, hi = vmax + 1u;  // mass(>= lo) >= p holds up to rounding; hi fails
  uint32_t c_lo = n_nz, c_hi = 0u;  // weights >= lo, weights >= hi
  double m_hi = 0.0;                 // mass of the weights >= hi
  {
    // first level: the bin where the mass counted from the top reaches p (a prefix sum over the
    // bins from the largest down; thread t holds bins 4095 - 4t - k, k < 4, in that order).
    // Rounding may leave p just past the total, and then the bisection starts from the whole range.
    const uint64_t MASK = (1ull << 48) - 1ull;
    const uint64_t p_fx = (uint64_t)ldexp(p_f64, WS_MASS_BITS);
    const int bin0 = WS_BINS - 1 - BPT * (int)threadIdx.x;
    uint64_t v[BPT], cum[BPT];
    uint64_t tsum = 0ull;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      v[k] = s_hist[bin0 - k];
      tsum += v[k];
      cum[k] = tsum;  // inclusive, inside the thread
    }
    const uint64_t sc = gp::wave_scan_u64(tsum);
    if (lane == 63) s_wtot[w] = sc;
    __syncthreads();
    uint64_t pre = 0ull;
    for (int k = 0; k < w; ++k) pre += s_wtot[k];
    pre += sc - tsum;  // before this thread's first bin
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const uint64_t incl = pre + cum[k], excl = incl - v[k];
      if ((excl & MASK) < p_fx && (incl & MASK) >= p_fx) {
        s_bin = bin0 - k;
        s_bin_incl = incl;
        s_bin_excl = excl;
      }
    }
    __syncthreads();
    const int b0 = gp::uni(s_bin);
    if (b0 >= 0) {
      const uint64_t bi = gp::uni((uint64_t)s_bin_incl), be = gp::uni((uint64_t)s_bin_excl);
      lo = max(1u, (uint32_t)b0 << WS_BIN_SHIFT);
      hi = min(vmax + 1u, ((uint32_t)b0 + 1u) << WS_BIN_SHIFT);
      c_hi = (uint32_t)(be >> 48);
      c_lo = (uint32_t)(bi >> 48);
      m_hi = ldexp((double)(be & MASK), -WS_MASS_BITS);
    }
  }
  while (hi - lo > 1u && c_lo - c_hi > (uint32_t)WS_TAIL) {
    const uint32_t mid = lo + (hi - lo) / 2;
    float s4[4] = {0.f, 0.f, 0.f, 0.f};
    uint32_t cm = 0u;
    each([&](int j) {
      const bool ge = u[j] >= mid;
      s4[j & 3] += ge ? __uint_as_float(u[j]) : 0.f;
      cm += ge;
    });
    uint32_t c_mid;
    const double sm = sum_dc((double)(s4[0] + s4[1]) + (double)(s4[2] + s4[3]), cm, &c_mid);
    if (sm >= p_f64) {
      lo = mid;
      c_lo = c_mid;
    } else {
      hi = mid;
      c_hi = c_mid;
      m_hi = sm;
    }
  }
  if (hi - lo > 1u) {
    // at most WS_TAIL weights in [lo, hi): list them; one wave sorts the list (descending) and
    // takes the first weight at which the running mass, from the mass at or above hi, reaches p
    static_assert(WS_TAIL == WS_TK * GP_WAVE, "the tail sort holds WS_TK keys per lane");
    __shared__ uint32_t s_tail[WS_TAIL];
    __shared__ uint32_t s_ntail, s_lo;
    if (threadIdx.x == 0) s_ntail = 0u;
    __syncthreads();
    each([&](int j) {
      const bool in = u[j] >= lo && u[j] < hi;
      const uint64_t m = __builtin_amdgcn_ballot_w64(in);
      if (m == 0) return;
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&s_ntail, (uint32_t)__builtin_popcountll(m));
      base = __shfl(base, 0, GP_WAVE);
      const uint32_t k = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (in && k < (uint32_t)WS_TAIL) s_tail[k] = u[j];
    });
    __syncthreads();
    if (w == 0) {
      const uint32_t nt = min(s_ntail, (uint32_t)WS_TAIL);  // == c_lo - c_hi <= WS_TAIL
      uint32_t xs[WS_TK];
#pragma unroll
      for (int k = 0; k < WS_TK; ++k) {
        const uint32_t idx = lane + GP_WAVE * k;
        xs[k] = idx < nt ? s_tail[idx] : 0u;  // empty places sort last
      }
      bitonic_sort_desc<WS_TAIL, WS_TK>(xs, lane);
      // inclusive running mass in sorted order; no crossing (rounding) keeps lo
      double run = m_hi;
      uint32_t found = lo;
      bool hit_any = false;
#pragma unroll
      for (int k = 0; k < WS_TK; ++k) {
        const double c = run + gp::wave_scan_f64((double)__uint_as_float(xs[k]));
        const uint64_t hit = __builtin_amdgcn_ballot_w64(xs[k] != 0u && c >= p_f64);
        if (!hit_any && hit != 0ull) {
          found = (uint32_t)__builtin_amdgcn_readlane((int)xs[k], (int)__builtin_ctzll(hit));
          hit_any = true;
        }
        run = __builtin_bit_cast(double, gp::readlane63_u64(__builtin_bit_cast(uint64_t, c)));
      }
      if (lane == 0) s_lo = found;
    }
    __syncthreads();
    lo = gp::uni(s_lo);
  }
  // snap T to the largest present weight <= lo
  uint32_t T;
  {
    uint32_t best = 0u;
    each([&](int j) { if (u[j] <= lo) best = max(best, u[j]); });
    T = max_x(best);
  }
  // next smaller / next larger weight value present in the row
  auto below_T = [&](uint32_t T0) {
    uint32_t best = 0u;
    each([&](int j) { if (u[j] < T0) best = max(best, u[j]); });
    return max_x(best);
  };
  auto above_T = [&](uint32_t T0) {
    uint32_t best = 0u;
    each([&](int j) { if (u[j] > T0) best = max(best, ~u[j]); });
    return ~max_x(best);
  };
  // certificate: mass(> T) < p <= mass(>= T); move T to a neighbour value until it holds. The
  // float64 sums, with their rounding bound, decide it and K = #(> T) + ceil((p - mass(> T)) / T)
  // whenever the bound leaves no doubt; otherwise the exact 160-bit sums below do.
  for (int iter = 0; iter < 64; ++iter) {
    {
      double gs = 0.0;
      // #(> T) << 16 | #(== T): each at most 32768 over the block (with T = 0 the empty slots
      // count as equal, which nothing below uses: the mass at T is then 0)
      uint32_t cc = 0;
      each([&](int j) {
        if (u[j] > T) {
          gs += (double)__uint_as_float(u[j]);
          cc += 1u << 16;
        } else if (u[j] == T) {
          cc += 1u;
        }
      });
      uint32_t cnt;
      const double mgt_f = sum_dc(gs, cc, &cnt);
      const uint32_t n_gt = cnt >> 16, n_eq = cnt & 0xffffu;
      const double Tf = (double)__uint_as_float(T);
      const double e_gt = SUM_ERR * mgt_f;
      const double mge_f = mgt_f + (double)n_eq * Tf;  // the product is exact: one rounding
      const double e_ge = e_gt + 0x1p-52 * mge_f;
      if (T != 0u && mge_f + e_ge < p_f64) {  // mass(>= T) < p: too high
        T = below_T(T);
        continue;
      }
      if (mgt_f - e_gt >= p_f64) {             // mass(> T) >= p: too low
        T = above_T(T);
        continue;
      }
      if (T != 0u && mge_f - e_ge >= p_f64 && mgt_f + e_gt < p_f64) {
        // X = (p - mass(> T)) / T in (0, #(== T)]: its ceiling is certain when no integer lies
        // within the bound of X
        const double X = (p_f64 - mgt_f) / Tf;
        const double eX = 2.0 * ((e_gt + 0x1p-53 * (p_f64 - mgt_f)) / Tf + 0x1p-52 * X);
        const double k1 = ceil(X - eX), k2 = ceil(X + eX);
        if (k1 == k2) {
          if (threadIdx.x == 0) *out = (int32_t)(n_gt + (uint32_t)max(1.0, k1));
          return;
        }
      }
    }
    Acc5 gt = {};
    uint32_t cgt = 0, ceq = 0;
#pragma unroll 4
    for (int j = 0; j < WS_VPT; ++j) {
      if (j >= nv) continue;
      if (u[j] > T) {
        acc_add(gt, u[j]);
        ++cgt;
      } else if (u[j] == T) {
        ++ceq;
      }
    }
    uint64_t t[8] = {gt.d[0], gt.d[1], gt.d[2], gt.d[3], gt.d[4], gt.d[5], (uint64_t)cgt, (uint64_t)ceq};
    sum_u8(t);
    Acc5 sgt;
#pragma unroll
    for (int k = 0; k < 6; ++k) sgt.d[k] = t[k];
    cgt = (uint32_t)t[6];
    ceq = (uint32_t)t[7];
    uint32_t mge[6], mgt[6];
    acc_norm(sgt, mgt);
    Acc5 sge = sgt;  // mass(>= T) = mass(> T) + #(== T) * T
    acc_add_mul(sge, T, ceq);
    acc_norm(sge, mge);
    if (T != 0u && cmp_p(mge, P.p_fixed) < 0) {  // too high: next smaller present value
      T = below_T(T);
      continue;
    }
    if (cmp_p(mgt, P.p_fixed) >= 0) {  // too low: next larger present value
      T = above_T(T);
      continue;
    }
    // K = #(> T) + ceil((p - mass(> T)) / T), all exact
    if (threadIdx.x == 0) {
      // X = p - mass(> T), 160-bit
      uint32_t X[5];
      int64_t borrow = 0;
      for (int k = 0; k < 5; ++k) {
        int64_t tk = (int64_t)P.p_fixed[k] - (int64_t)mgt[k] - borrow;
        borrow = tk < 0;
        X[k] = (uint32_t)(tk + (borrow ? 4294967296ll : 0ll));
      }
      const uint32_t E = T >> 23;
      uint32_t M = T & 0x7fffffu, sh = 0;
      if (E) {
        M |= 0x800000u;
        sh = E - 1u;
      }
      // Y = X >> sh (fits 64 bits), and whether any shifted-out bit was set
      const uint32_t w0 = sh >> 5, o = sh & 31u;
      uint64_t Y = 0;
      bool rem = false;
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        const uint64_t xk = X[k];
        if ((uint32_t)k < w0) rem |= xk != 0u;
        if ((uint32_t)k == w0) rem |= (o ? (xk & ((1ull << o) - 1ull)) : 0ull) != 0ull;
        const int rel = k - (int)w0;  // word k lands at bit 32*rel - o of Y
        if (rel >= 0 && rel <= 2) {
          const int at = 32 * rel - (int)o;
          Y |= at >= 0 ? (xk << at) : (xk >> (-at));
        }
      }
      uint64_t j = Y / M;
      if (rem || (Y % M) != 0ull) ++j;
      if (j == 0) j = 1;
      *out = (int32_t)(cgt + j);
    }
    return;
  }
  if (threadIdx.x == 0) *out = -2;  // certificate did not converge (not expected)
}

}  // namespace

// p as a 160-bit fixed-point number of 2^-149 units, rounded up (so "sum >= p" is exact)
static void p_to_fixed(double p, uint32_t out[5]) {
  for (int k = 0; k < 5; ++k) out[k] = 0;
  int e;
  const double m = frexp(p, &e);  // p = m * 2^e, m in [0.5, 1)
  const uint64_t mant = (uint64_t)ldexp(m, 53);  // p = mant * 2^(e - 53)
  const int shift = e - 53 + 149;
  if (shift >= 0) {
    for (int bit = 0; bit < 53; ++bit)
      if ((mant >> bit) & 1ull) {
        const int b = bit + shift;
        if (b < 160) out[b >> 5] |= 1u << (b & 31);
      }
  } else {
    const int s = -shift;
    uint64_t q = s >= 64 ? 0 : (mant >> s);
    const bool r = s >= 64 ? mant != 0 : (mant & ((1ull << s) - 1)) != 0;
    if (r) ++q;
    out[0] = (uint32_t)q;
    out[1] = (uint32_t)(q >> 32);
  }
}

extern "C" size_t gp_score_and_working_set_workspace_size(int R, int H_q, int H_kv, int head_dim,
                                                          int page_size, int C_max) {
  (void)H_kv;
  (void)page_size;
  if (R <= 0 || H_q <= 0 || head_dim <= 0 || C_max <= 0) return 0;
  const size_t nch = (C_max + CHUNK_TILES * 16 - 1) / (CHUNK_TILES * 16);
  const size_t c_pad = (size_t)((C_max + 3) / 4) * 4;
  return ((size_t)R * 2 * H_q * c_pad + (size_t)R * 2 * H_q * nch * 2) * sizeof(float);
}

extern "C" int gp_score_and_working_set(const void* q, int q_dtype, int B, int H_q, const float* qstate,
                                        int num_slots, const int32_t* slot_ids, const int32_t* req_idx,
                                        int R, const gp_kv_cache* kv, const int32_t* block_tables,
                                        int max_pages, const int32_t* context_lens,
                                        const int32_t* positions, float rope_theta, double p,
                                        float sm_scale, float* a_short, float* a_long, int C_max,
                                        int32_t* ws_counts, int32_t* n_cand, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  if (R < 0 || B < 0 || H_q <= 0 || num_slots <= 0 || !kv || max_pages <= 0 || C_max <= 0)
    return GP_ERR_INVALID;
  if (R == 0) return GP_OK;
  if (!q || !qstate || !slot_ids || !req_idx || !block_tables || !context_lens || !positions ||
      !a_short || !a_long || !ws_counts || !n_cand || !kv->k)
    return GP_ERR_INVALID;
  if (!(p > 0.0 && p <= 1.0)) return GP_ERR_INVALID;
  const int H_kv = kv->num_kv_heads, D = kv->head_dim, b = kv->page_size;
  if (H_kv <= 0 || H_q % H_kv != 0 || kv->num_pages <= 0) return GP_ERR_INVALID;
  if (q_dtype != kv->dtype || (q_dtype != GP_F32 && q_dtype != GP_BF16)) return GP_ERR_INVALID;
  if (kv->page_tag) {
    // mixed-precision pages: bf16 caches with the fp8 and INT4 key pools
    if (kv->dtype != GP_BF16) return GP_ERR_UNSUPPORTED;
    if (!kv->k8 || !kv->k_scale || !kv->k4 || !kv->k4_scale) return GP_ERR_INVALID;
  }
  if (D != 64 && D != 128) return GP_ERR_UNSUPPORTED;
  if (b < 16 || b > 256 || b % 16) return GP_ERR_UNSUPPORTED;
  const int G = H_q / H_kv;
  if (2 * G > 16) return GP_ERR_UNSUPPORTED;
  if (C_max > WS_MAX_C || C_max % 4) return GP_ERR_UNSUPPORTED;
  const size_t need = gp_score_and_working_set_workspace_size(R, H_q, H_kv, D, b, C_max);
  if (!workspace || workspace_bytes < need) return GP_ERR_WORKSPACE;

  ScoreParams P{};
  P.q = q;
  P.qstate = qstate;
  P.slot_ids = slot_ids;
  P.req_idx = req_idx;
  P.k = kv->k;
  P.page_tag = kv->page_tag;
  P.k8 = static_cast<const uint8_t*>(kv->k8);
  P.k_scale = kv->k_scale;
  P.k4 = static_cast<const uint8_t*>(kv->k4);
  P.k4_scale = kv->k4_scale;
  P.block_tables = block_tables;
  P.context_lens = context_lens;
  P.positions = positions;
  P.a_short = a_short;
  P.a_long = a_long;
  P.ws_counts = ws_counts;
  P.n_cand = n_cand;
  P.B = B;
  P.R = R;
  P.H_q = H_q;
  P.H_kv = H_kv;
  P.G = G;
  P.D = D;
  P.page_size = b;
  P.num_pages = kv->num_pages;
  P.max_pages = max_pages;
  P.num_slots = num_slots;
  P.C_max = C_max;
  P.nch = (C_max + CHUNK_TILES * 16 - 1) / (CHUNK_TILES * 16);
  P.q_bf16 = q_dtype == GP_BF16;
  P.scale_log2 = sm_scale * GP_LOG2E;
  P.rope_theta = rope_theta;
  for (int j = 0; j < 64; ++j)
    P.inv_freq[j] = (rope_theta > 0.f && j < D / 2) ? std::pow((double)rope_theta, -2.0 * j / D) : 0.0;
  p_to_fixed(p, P.p_fixed);
  float* ws = static_cast<float*>(workspace);
  P.logits = ws;
  P.stats = P.logits + (size_t)R * 2 * H_q * (size_t)((C_max + 3) / 4) * 4;

  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 lg(H_kv, P.nch, R);
  const dim3 lt(((long)H_kv * P.nch * R <= LG_FEW_WORKGROUPS ? LG_MAX_WAVES : LG_MIN_WAVES) * GP_WAVE);
  if (kv->page_tag) {  // mixed caches are bf16 (checked above)
    if (D == 64) hipLaunchKernelGGL((logits_kernel<64, true, true>), lg, lt, 0, s, P);
    else hipLaunchKernelGGL((logits_kernel<128, true, true>), lg, lt, 0, s, P);
  } else if (q_dtype == GP_BF16) {
    if (D == 64) hipLaunchKernelGGL((logits_kernel<64, true, false>), lg, lt, 0, s, P);
    else hipLaunchKernelGGL((logits_kernel<128, true, false>), lg, lt, 0, s, P);
  } else {
    if (D == 64) hipLaunchKernelGGL((logits_kernel<64, false, false>), lg, lt, 0, s, P);
    else hipLaunchKernelGGL((logits_kernel<128, false, false>), lg, lt, 0, s, P);
  }
  GP_CHECK_LAUNCH();
  hipLaunchKernelGGL(working_set_kernel, dim3(2 * H_kv, R), dim3(WS_THREADS), 0, s, P);
  GP_CHECK_LAUNCH();
  return GP_OK;
}
