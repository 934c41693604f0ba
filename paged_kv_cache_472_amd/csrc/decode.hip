// Paged decode attention for gfx950 (PASK Sec. 3.1 attention definition, App. B.5 split-KV
// merge and mixed-precision page reads; GrowPage Sec. 4.2 block tables).
//
// Work decomposition (stream-K over a variable-length batch): the (request, 16-token tile) units
// of the whole batch are laid end to end and cut into equal contiguous ranges, one per resident
// workgroup, so every compute unit streams the same number of bytes whatever the length mix.
// A workgroup holds one wave64 per KV head (up to 8); all its waves walk the same tiles, so
// together they read each page's whole K block and V block (the heads of a page are adjacent
// in HBM). A range that covers a whole request writes its output directly; otherwise each
// request segment leaves a partial (max, sum, unnormalised output) that a second kernel merges
// with the rule of PASK App. B.5.
//
// Per tile the G query heads of the wave's KV head are contracted against the key tile on the
// matrix cores (keys as the 16-row operand, heads as the 16-column operand, so the result lands
// with one head per lane column), an online softmax runs on the 4 logits each lane holds, and the
// probability tile - already in the operand layout of the next product - is multiplied with the
// value tile (values are stored token-contiguous inside a page, so each lane reads 4 consecutive
// tokens of one value row). Each wave first lists, in its own LDS region, the tiles of up to 256
// at a time that the pass decodes (page code and tile index, skipped pages left out; the first
// pass over a mixed cache keeps its bf16 and its fp8 tiles in two lists, each walked with the
// format fixed at compile time), then walks the list with a register ring whose slots rotate by
// unrolling. Every ring slot is refilled
// unconditionally (past the end with the last entry again, never processed): with loads that
// depend on no branch, the wait before a tile's products covers that tile's own loads and not
// the ones issued after it, so the ring's depth is what stays in flight per wave.
//
// Mixed-precision caches decode in two passes over the same batch, each leaving partials that
// the merge combines: the first takes the bf16 and fp8 tiles, the second the INT4 tiles with an
// INT4-only kernel (16 registers per tile, three tiles in flight per wave, its own stream-K width). Released
// pages are skipped, fp8 codes are widened exactly to bf16 and their row scales applied to the
// logits and the probability weights, and INT4 pages (PASK App. B.5) are contracted in half
// precision: their nibbles become exact half values through the mantissa of 1024.0. An INT4
// tile is five loads per lane: the lane's quarter of a key row (the key product pairs it with a
// half copy of the query holding the same dimensions, in the order the nibbles unpack in), the
// lane's head_dim/16 value dimensions of its four tokens (adjacent in the stored value block),
// and the four key and value half scales of its tokens. The value product takes the four tokens
// in the order (0, 2, 1, 3) on both operands. The online softmax rescales lazily: the running
// maximum moves only when a logit exceeds it by more than 2^8, so most tiles skip the rescale.
#include "common.h"

#include <algorithm>
#include <atomic>

namespace {

constexpr int KIND_F32 = 0;
constexpr int KIND_BF16 = 1;
constexpr int KIND_MIXED = 2;  // first pass over a mixed cache: its bf16 tiles, then its fp8 tiles
constexpr int KIND_INT4 = 3;   // a mixed cache's INT4 tiles only (the second pass)
constexpr int KIND_FP8 = 4;    // the fp8 tiles of the first pass over a mixed cache (narrow tiles)
// Tiles in flight per wave over a list of fp8 tiles: an fp8 tile holds half the registers and
// half the bytes of a bf16 one, so the same registers keep twice as many in flight.
constexpr int RING_FP8 = 4;
// The INT4 pass (16 registers per tile): three tiles in flight per wave (measured: two 0.184 ms,
// three 0.175 ms, four 0.193 ms for the Qwen3-8B-shaped batch with every page INT4).
constexpr int RING_INT4 = 3;
constexpr int MAX_HEADS_PER_WG = 8;
constexpr int MAX_THREADS = MAX_HEADS_PER_WG * GP_WAVE;
// Tiles in flight per wave (the register ring's depth). Two keep HBM busiest when the decode has
// the GPU to itself. A call with a workgroup cap is meant to share the GPU with latency-bound
// kernels (a boundary pass): there the bf16 / fp32 decode keeps one, because deeper memory queues
// slow every dependent access of the kernels beside it far more than they speed up the decode.
constexpr int RING_FULL = 2;
constexpr int RING_SHARED = 1;
// The INT4 pass is bound by instruction issue, not bytes (about twice the VALU instructions of a
// bf16 tile for a quarter of the bytes): its kernel (168 registers) runs three waves per SIMD, in
// workgroups of four heads, so that more of them share a compute unit than eight-head ones would.
constexpr int INT4_HEADS_PER_WG = 4;
constexpr int MAX_BATCH = 8191;   // prefix of tile counts kept in LDS (32 KB)
constexpr int LIST = 256;         // tiles per wave listed in LDS at a time

// LDS ints of the prefix of tile counts, rounded up so that the tile lists start 16-byte aligned
__host__ __device__ __forceinline__ int pref_ints(int B) { return (B + 1 + 3) & ~3; }
constexpr int J_CAP_MAX = 127;    // partials one output row can have (the merge holds two per lane)

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const uint8_t* k8;
  const uint8_t* v8;
  const float* k_scale;
  const float* v_scale;
  const uint8_t* k4;
  const uint8_t* v4;
  const uint16_t* k4_scale;
  const uint16_t* v4_scale;
  const uint8_t* page_tag;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse;
  float* ws_o;       // [B, H_q, passes * J_max, D] partial outputs
  float* ws_ml;      // [B, H_q, passes * J_max, 2] partial (max, sum)
  int32_t* ws_pref;  // [B + 1] prefix of tile counts, written by workgroup 0
  // fused summary update (NULL q_pre: none)
  const void* q_pre;
  const int32_t* slot_ids;
  const uint8_t* fresh;
  float* qstate;
  int num_slots;
  float beta_s, beta_l;
  int B, H_q, H_kv, G, page_size, num_pages, max_pages, max_context;
  int heads_per_wg;
  int passes;  // 2 for a mixed cache: the bf16 / fp8 tiles, then the INT4 tiles
  int pass;    // this launch's pass; its partials sit in slots pass * j_max + j
  int num_wg;  // workgroups per head group (the stream-K width) of this launch
  int num_wg_pass[2];  // the stream-K width of each pass (the merge needs both)
  int r_min;   // minimum tiles per range
  int j_max;   // partial slots per output row
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
struct TileRaw<D, KIND_FP8> {
  u32x2_t k[D / 32];   // 8 key codes of the row per 32-wide k step
  uint32_t v[D / 16];  // 4 codes (4 tokens) of one value row per 16-row block
  f32x4_t ks, vs;      // fp32 scales of the lane's 4 tokens
};

template <int D>
struct TileRaw<D, KIND_INT4> {
  u32x4_t k;             // the lane's D/4 key codes (D = 64: in .xy)
  u32x2_t v[D / 64];     // 2 bytes (4 tokens) for each of D/16 value dimensions
  f32x4_t ks, vs;        // the 4 half scales of the lane's tokens, in .xy
};

__device__ __forceinline__ int sanitize_ctx(const DecodeParams& p, int r) {
  int ctx = p.context_lens[r];
  const long cap = (long)p.max_pages * p.page_size;
  if (ctx < 0 || ctx > p.max_context || ctx > cap) ctx = 0;
  return ctx;
}

// The key and value halves of one INT4 tile (the walk over INT4 tiles refills them separately).
template <int D>
struct KRing4 {
  u32x4_t k;   // the lane's D/4 key codes (D = 64: in .xy)
  u32x2_t ks;  // the 4 half scales of the lane's tokens
};
template <int D>
struct VRing4 {
  u32x2_t v[D / 64];  // 2 bytes (4 tokens) for each of D/16 value dimensions
  u32x2_t vs;         // the 4 half scales of the lane's tokens
};

// Row index (page, KV head, first token of the tile) of an INT4 tile: wave-uniform, so the
// loads below take a scalar base plus a 32-bit lane offset. The lane offsets are made opaque per
// load; otherwise the compiler hoists pool + lane offset out of the tile loop as a 64-bit vector
// pointer and adds the page part to it with vector instructions on every tile.
__device__ __forceinline__ size_t int4_row0(const DecodeParams& p, int code, int tok0, int h) {
  return ((size_t)(code >> 2) * p.H_kv + h) * (size_t)p.page_size + tok0 % p.page_size;
}

template <int D>
__device__ __forceinline__ void load_k4(const DecodeParams& p, int code, int tok0, int h,
                                        int lane, KRing4<D>& t) {
  const int n16 = lane & 15, g4 = lane >> 4;
  const size_t row0 = int4_row0(p, code, tok0, h);
  uint32_t k_lane = (uint32_t)(n16 * (D / 2) + g4 * (D / 8));
  uint32_t s_lane = (uint32_t)(8 * g4);  // bytes: 4 half scales per lane
  asm volatile("" : "+v"(k_lane), "+v"(s_lane));
  const uint8_t* kb = p.k4 + row0 * (D / 2);
  if constexpr (D == 128)
    t.k = gp::ld_stream<u32x4_t>(kb + k_lane);
  else
    *reinterpret_cast<u32x2_t*>(&t.k) = gp::ld_stream<u32x2_t>(kb + k_lane);
  t.ks = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint8_t*>(p.k4_scale + row0) + s_lane);
}

template <int D>
__device__ __forceinline__ void load_v4(const DecodeParams& p, int code, int tok0, int h,
                                        int lane, VRing4<D>& t) {
  const int n16 = lane & 15, g4 = lane >> 4;
  const size_t row0 = int4_row0(p, code, tok0, h);
  uint32_t v_lane = (uint32_t)(g4 * (2 * D) + n16 * (D / 8));
  uint32_t s_lane = (uint32_t)(8 * g4);
  asm volatile("" : "+v"(v_lane), "+v"(s_lane));
  const uint8_t* vb = p.v4 + (row0 >> 2) * (2 * D);  // 4-token blocks of 2 D bytes
#pragma unroll
  for (int i = 0; i < D / 64; ++i) t.v[i] = *reinterpret_cast<const u32x2_t*>(vb + v_lane + 8 * i);
  t.vs = *reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint8_t*>(p.v4_scale + row0) + s_lane);
}

// Load tile `tok0` (a multiple of 16) of KV head h from the page encoded in `code`. Loads whose
// instruction covers whole 128-byte lines (value rows of bf16, fp32 and fp8 pages, INT4 key rows)
// are streaming loads; key rows read 64 bytes per row per instruction (the other half comes with
// the next instruction) and the scales keep ordinary loads: a streaming half line can leave the
// cache before its other half is read, and then the line is fetched twice.
template <int D, int KIND>
__device__ __forceinline__ void load_tile(const DecodeParams& p, int code, int tok0, int h,
                                          int lane, TileRaw<D, KIND>& t) {
  const int n16 = lane & 15, g4 = lane >> 4;
  const int b = p.page_size;
  const int off = tok0 % b;
  if constexpr (KIND == KIND_INT4) {
    KRing4<D> kh;
    VRing4<D> vh;
    load_k4<D>(p, code, tok0, h, lane, kh);
    load_v4<D>(p, code, tok0, h, lane, vh);
    t.k = kh.k;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) t.v[i] = vh.v[i];
    *reinterpret_cast<u32x2_t*>(&t.ks) = kh.ks;
    *reinterpret_cast<u32x2_t*>(&t.vs) = vh.vs;
  } else if constexpr (KIND == KIND_FP8) {
    const int pg = code;
    const size_t kv_base = ((size_t)pg * p.H_kv + h) * (size_t)b * D;
    const size_t sb = ((size_t)pg * p.H_kv + h) * b + off + 4 * g4;
    const uint8_t* kr = p.k8 + kv_base + (size_t)(off + n16) * D + 8 * g4;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = *reinterpret_cast<const u32x2_t*>(kr + 32 * kk);
    const uint8_t* vr = p.v8 + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = gp::ld_stream<uint32_t>(vr + (size_t)16 * nb * b);
    t.ks = *reinterpret_cast<const f32x4_t*>(p.k_scale + sb);
    t.vs = *reinterpret_cast<const f32x4_t*>(p.v_scale + sb);
  } else {
    const size_t kv_base = ((size_t)code * p.H_kv + h) * (size_t)b * D;
    if constexpr (KIND == KIND_BF16) {
      const uint16_t* kr = reinterpret_cast<const uint16_t*>(p.k) + kv_base + (size_t)(off + n16) * D + 8 * g4;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) t.k[kk] = *reinterpret_cast<const u32x4_t*>(kr + 32 * kk);
      const uint16_t* vr = reinterpret_cast<const uint16_t*>(p.v) + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = gp::ld_stream<u32x2_t>(vr + (size_t)16 * nb * b);
    } else {
      const float* kr = reinterpret_cast<const float*>(p.k) + kv_base + (size_t)(off + n16) * D + (D / 4) * g4;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) t.k[i] = *reinterpret_cast<const u32x4_t*>(kr + 4 * i);
      const float* vr = reinterpret_cast<const float*>(p.v) + kv_base + (size_t)n16 * b + off + 4 * g4;
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) t.v[nb] = gp::ld_stream<u32x4_t>(vr + (size_t)16 * nb * b);
    }
  }
}

// Running softmax state of one wave: output rows of the G heads (acc, head 4*g4 + i in
// component i, dim 16*nb + n16), running max (log2 domain) of head n16, this lane's share of the
// running sum of head n16.
template <int D>
struct WaveState {
  f32x4_t acc[D / 16];
  float m_run, l_run;
};

// TAIL: the tile holds the request's last token (tok0 + 16 > ctx), so some of its tokens lie past
// the context and are masked. Only such a tile needs the masks and the guards against -inf logits
// (every token of another tile is live, so its logits and the running maximum are finite); the
// walk branches between the two forms once per tile.
template <int D, int KIND, bool TAIL>
__device__ __forceinline__ void process_tile(const DecodeParams& p, const TileRaw<D, KIND>& cur,
                                             int tok0, int ctx, int lane,
                                             const u32x4_t* qf, const f16x8_t* qh,
                                             WaveState<D>& st) {
  const int g4 = lane >> 4;
  constexpr bool tail = TAIL;
  // per-token scales of the lane's 4 tokens (fp8: fp32 values; INT4: halves)
  constexpr bool SCALED = KIND == KIND_INT4 || KIND == KIND_FP8;
  float ks[4], vs[4];
  if constexpr (KIND == KIND_INT4) {
    const uint32_t k01 = __float_as_uint(cur.ks[0]), k23 = __float_as_uint(cur.ks[1]);
    const uint32_t v01 = __float_as_uint(cur.vs[0]), v23 = __float_as_uint(cur.vs[1]);
    ks[0] = gp::half_lo(k01); ks[1] = gp::half_hi(k01); ks[2] = gp::half_lo(k23); ks[3] = gp::half_hi(k23);
    vs[0] = gp::half_lo(v01); vs[1] = gp::half_hi(v01); vs[2] = gp::half_lo(v23); vs[3] = gp::half_hi(v23);
  } else if constexpr (KIND == KIND_FP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { ks[i] = cur.ks[i]; vs[i] = cur.vs[i]; }
  }
  // ---- logits: S[token 4*g4 + i][head n16]
  f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KIND == KIND_INT4) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      sacc = gp::mfma_f16_16x16x32(gp::int4x8_to_f16x8(cur.k[kk]), qh[kk], sacc);
  } else if constexpr (KIND == KIND_F32) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sacc = gp::mfma_f32_16x16x4(__uint_as_float(cur.k[i][c]), __uint_as_float(qf[i][c]), sacc);
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      u32x4_t kw;
      if constexpr (KIND == KIND_FP8) {
        // fp8 codes widen exactly to bf16
        const u32x2_t lo = gp::fp8x4_to_bf16x4(cur.k[kk].x), hi = gp::fp8x4_to_bf16x4(cur.k[kk].y);
        kw = u32x4_t{lo.x, lo.y, hi.x, hi.y};
      } else {
        kw = cur.k[kk];
      }
      sacc = gp::mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, kw),
                                    __builtin_bit_cast(bf16x8_t, qf[kk]), sacc);
    }
  }
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float z = sacc[i];
    if constexpr (SCALED) z *= ks[i];
    sv[i] = z * p.scale_log2;
    if constexpr (TAIL)
      if (tok0 + 4 * g4 + i >= ctx) sv[i] = -INFINITY;
  }
  float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mx = gp::xor16_max(mx);
  mx = gp::xor32_max(mx);
  // lazy rescaling: the running maximum moves only when a logit exceeds it by more than 2^8
  // (log2 domain 8), so the weights stay below 256 and most tiles skip the rescale of the rows
  const bool move = mx > st.m_run + 8.0f;
  const float m_new = move ? mx : st.m_run;
  const float alpha = move ? gp::safe_exp2_diff(st.m_run, m_new) : 1.0f;
  float pv[4];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // outside a tail tile the logits and m_new are finite (m_new >= this tile's maximum)
    pv[i] = TAIL ? gp::safe_exp2_diff(sv[i], m_new) : __builtin_amdgcn_exp2f(sv[i] - m_new);
    psum += pv[i];
  }
  st.l_run = st.l_run * alpha + psum;
  st.m_run = m_new;
  if (__builtin_amdgcn_ballot_w64(move) != 0) {
    // rescale the output rows: this lane holds heads 4*g4 + i
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g4 + i, GP_WAVE);
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[nb][i] *= al[i];
  }
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
      for (int i = 0; i < 4; ++i) st.acc[nb] = gp::mfma_f32_16x16x4(pv[i], __uint_as_float(vw[i]), st.acc[nb]);
    }
  } else {
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = pv[i];
      if constexpr (SCALED) {
        pw[i] *= vs[i];
        if constexpr (TAIL)
          if (pv[i] == 0.f) pw[i] = 0.f;  // scales of masked tokens may be poison
      }
    }
    if constexpr (KIND == KIND_INT4) {
      // every INT4 byte decodes to a finite code, so no value masking is needed
      const f16x2_t p02 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(pw[0], pw[2]));
      const f16x2_t p13 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(pw[1], pw[3]));
      const f16x4_t ph = f16x4_t{p02.x, p02.y, p13.x, p13.y};
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        const uint32_t word = cur.v[nb / 4][(nb / 2) % 2];  // dimension 16 nb + n16: 2 bytes
        const uint32_t grp = (nb % 2) ? (word >> 16) : word;
        st.acc[nb] = gp::mfma_f16_16x16x16(ph, gp::int4x4_to_f16x4(grp), st.acc[nb]);
      }
    } else {
      const u32x2_t pp = u32x2_t{gp::pack_bf16x2(pw[0], pw[1]), gp::pack_bf16x2(pw[2], pw[3])};
      // values of tokens past the context (the tail of the last page) are masked to zero bits
      uint32_t mlo = 0xffffffffu, mhi = 0xffffffffu;
      if (tail) {
        const int base = tok0 + 4 * g4;
        mlo = (base + 0 < ctx ? 0x0000ffffu : 0u) | (base + 1 < ctx ? 0xffff0000u : 0u);
        mhi = (base + 2 < ctx ? 0x0000ffffu : 0u) | (base + 3 < ctx ? 0xffff0000u : 0u);
      }
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        u32x2_t vw;
        if constexpr (KIND == KIND_FP8)
          vw = gp::fp8x4_to_bf16x4(cur.v[nb]);
        else
          vw = cur.v[nb];
        vw.x &= mlo;
        vw.y &= mhi;
        st.acc[nb] = gp::mfma_bf16_16x16x16(__builtin_bit_cast(i16x4_t, pp),
                                            __builtin_bit_cast(i16x4_t, vw), st.acc[nb]);
      }
    }
  }
}


// Walk n listed tiles (page codes and tile indexes in LDS) with a register ring of RING tiles.
// Every slot is refilled unconditionally (past the end of the list with the last entry again,
// which is never processed), so each iteration issues the same loads and the wait before a tile's
// products covers only that tile's loads. Every listed page has the format KIND decodes, so no
// load depends on a branch either.
template <int D, int KIND, int RING>
__device__ __forceinline__ void walk_tiles(const DecodeParams& p, const int* lst_code,
                                           const int* lst_tile, int n, int h, int lane, int ctx,
                                           const u32x4_t* qf, const f16x8_t* qh, WaveState<D>& st) {
  if (n == 0) return;
  TileRaw<D, KIND> ring[RING];
  int rc[RING], rt[RING];
#pragma unroll
  for (int q = 0; q < RING; ++q) {
    const int e = min(q, n - 1);
    rc[q] = __builtin_amdgcn_readfirstlane(lst_code[e]);
    rt[q] = __builtin_amdgcn_readfirstlane(lst_tile[e]);
    load_tile<D, KIND>(p, rc[q], rt[q] << 4, h, lane, ring[q]);
  }
  // only the list's last tile can hold the request's last token: the loop decodes every other
  // tile without masks, and that one, if it is a tail tile, after the loop (its ring slot then
  // holds it again: slots past the end reload the last entry)
  // (fp32 caches, used for small checks only, keep one tile form: their registers are tight)
  constexpr bool SPLIT = KIND != KIND_F32;
  const int last_tok0 = __builtin_amdgcn_readfirstlane(lst_tile[n - 1]) << 4;
  const bool has_tail = SPLIT && last_tok0 + 16 > ctx;
  const int n_main = has_tail ? n - 1 : n;
  for (int e0 = 0; e0 < n; e0 += RING) {
#pragma unroll
    for (int q = 0; q < RING; ++q) {
      const int e = e0 + q;
      if (e < n_main) process_tile<D, KIND, !SPLIT>(p, ring[q], rt[q] << 4, ctx, lane, qf, qh, st);
      const int ex = min(e + RING, n - 1);
      rc[q] = __builtin_amdgcn_readfirstlane(lst_code[ex]);
      rt[q] = __builtin_amdgcn_readfirstlane(lst_tile[ex]);
      load_tile<D, KIND>(p, rc[q], rt[q] << 4, h, lane, ring[q]);
    }
  }
  if (SPLIT && has_tail) {
    const int slot = (n - 1) % RING;
#pragma unroll
    for (int q = 0; q < RING; ++q)
      if (q == slot) process_tile<D, KIND, true>(p, ring[q], last_tok0, ctx, lane, qf, qh, st);
  }
}

// Walk n listed INT4 tiles in turns of RING_INT4 tiles, with the softmax bookkeeping once per
// turn: the logits of the turn's tiles, one cross-lane maximum and one (rare) rescale of the
// output rows for all of them, then their weighted values. A key slot is refilled right after its
// logits and a value slot right after its products, so each wait covers one half tile. Slots past
// the list's main part (its end, or a tail tile, which is decoded after the loop with its masks)
// go through the same instructions as no-ops: their logits stay out of the maximum and their
// weights are zero (INT4 codes are always finite, so zero weights leave the rows unchanged).
// Why per turn: the per-tile rescale branch made the compiler copy all 32 output registers on
// every tile's common path; here the bookkeeping and any such copies come once per turn.
template <int D>
__device__ __forceinline__ void walk_tiles_int4(const DecodeParams& p, const int* lst_code,
                                                const int* lst_tile, int n, int h, int lane,
                                                int ctx, const f16x8_t* qh, WaveState<D>& st) {
  constexpr int RING = RING_INT4;
  if (n == 0) return;
  const int g4 = lane >> 4;
  KRing4<D> kr[RING];
  VRing4<D> vr[RING];
#pragma unroll
  for (int q = 0; q < RING; ++q) {
    const int e = min(q, n - 1);
    const int c = __builtin_amdgcn_readfirstlane(lst_code[e]);
    const int t = __builtin_amdgcn_readfirstlane(lst_tile[e]) << 4;
    load_k4<D>(p, c, t, h, lane, kr[q]);
    load_v4<D>(p, c, t, h, lane, vr[q]);
  }
  const int last_tok0 = __builtin_amdgcn_readfirstlane(lst_tile[n - 1]) << 4;
  const bool has_tail = last_tok0 + 16 > ctx;
  const int n_main = has_tail ? n - 1 : n;
  for (int e0 = 0; e0 < n; e0 += RING) {
    // ---- logits of the turn's tiles: S[token 4*g4 + i][head n16], log2 domain
    float sv[RING][4];
    float tmax = -INFINITY;
    int nc[RING], nt[RING];  // the entry each slot is refilled with (keys now, values below)
#pragma unroll
    for (int q = 0; q < RING; ++q) {
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk)
        sacc = gp::mfma_f16_16x16x32(gp::int4x8_to_f16x8(kr[q].k[kk]), qh[kk], sacc);
      sv[q][0] = gp::mul_half_lo(sacc[0], kr[q].ks.x) * p.scale_log2;
      sv[q][1] = gp::mul_half_hi(sacc[1], kr[q].ks.x) * p.scale_log2;
      sv[q][2] = gp::mul_half_lo(sacc[2], kr[q].ks.y) * p.scale_log2;
      sv[q][3] = gp::mul_half_hi(sacc[3], kr[q].ks.y) * p.scale_log2;
      const float m4 = fmaxf(fmaxf(sv[q][0], sv[q][1]), fmaxf(sv[q][2], sv[q][3]));
      tmax = e0 + q < n_main ? fmaxf(tmax, m4) : tmax;
      const int ex = min(e0 + q + RING, n - 1);
      nc[q] = __builtin_amdgcn_readfirstlane(lst_code[ex]);
      nt[q] = __builtin_amdgcn_readfirstlane(lst_tile[ex]) << 4;
      load_k4<D>(p, nc[q], nt[q], h, lane, kr[q]);
    }
    // ---- one running-maximum step for the turn (lazy: moves only by more than 2^8)
    float mx = gp::xor16_max(tmax);
    mx = gp::xor32_max(mx);
    const bool move = mx > st.m_run + 8.0f;
    const float m_new = move ? mx : st.m_run;
    const float alpha = move ? gp::safe_exp2_diff(st.m_run, m_new) : 1.0f;
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(move) != 0, 0)) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * g4 + i, GP_WAVE);
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[nb][i] *= al[i];
    }
    // ---- weighted values of the turn's tiles
    float psum = 0.f;
#pragma unroll
    for (int q = 0; q < RING; ++q) {
      const bool live = e0 + q < n_main;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(sv[q][i] - m_new);
      const float ps = (pv[0] + pv[1]) + (pv[2] + pv[3]);
      const float pw[4] = {gp::mul_half_lo(pv[0], vr[q].vs.x), gp::mul_half_hi(pv[1], vr[q].vs.x),
                           gp::mul_half_lo(pv[2], vr[q].vs.y), gp::mul_half_hi(pv[3], vr[q].vs.y)};
      psum += live ? ps : 0.f;
      // a no-op slot's weights may be NaN (its scales can be poison): the select clears them
      const uint32_t p02 = live ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[0], pw[2])) : 0u;
      const uint32_t p13 = live ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pw[1], pw[3])) : 0u;
      const f16x4_t ph = __builtin_bit_cast(f16x4_t, u32x2_t{p02, p13});
#pragma unroll
      for (int wd = 0; wd < D / 32; ++wd) {
        // dimensions 16 (2 wd) + n16 and 16 (2 wd + 1) + n16: 2 bytes each
        f16x4_t va, vb;
        gp::int4_word_to_f16x4x2(vr[q].v[wd / 2][wd % 2], va, vb);
        st.acc[2 * wd] = gp::mfma_f16_16x16x16(ph, va, st.acc[2 * wd]);
        st.acc[2 * wd + 1] = gp::mfma_f16_16x16x16(ph, vb, st.acc[2 * wd + 1]);
      }
      load_v4<D>(p, nc[q], nt[q], h, lane, vr[q]);
    }
    st.l_run = st.l_run * alpha + psum;
    st.m_run = m_new;
  }
  if (has_tail) {
    // slots past the end hold the last entry again
    const int slot = (n - 1) % RING;
#pragma unroll
    for (int q = 0; q < RING; ++q)
      if (q == slot) {
        TileRaw<D, KIND_INT4> t;
        t.k = kr[q].k;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) t.v[i] = vr[q].v[i];
        *reinterpret_cast<u32x2_t*>(&t.ks) = kr[q].ks;
        *reinterpret_cast<u32x2_t*>(&t.vs) = vr[q].vs;
        process_tile<D, KIND_INT4, true>(p, t, last_tok0, ctx, lane, nullptr, qh, st);
      }
  }
}

// LDS ints per wave for tile lists: page codes and tile indexes; a mixed cache's first pass keeps
// its bf16 and fp8 tiles in two lists.
template <int KIND>
constexpr int list_ints() { return (KIND == KIND_MIXED ? 4 : 2) * LIST; }

// Tiles per workgroup range: equal shares of the batch's U units, at least r_min.
__device__ __forceinline__ int range_len(int num_wg, int r_min, int U) {
  return max((U + num_wg - 1) / num_wg, r_min);
}
__device__ __forceinline__ int range_len(const DecodeParams& p, int U) {
  return range_len(p.num_wg, p.r_min, U);
}

template <int D, int KIND, int RING>
__global__ __launch_bounds__(MAX_THREADS) void decode_streamk_kernel(DecodeParams p) {
  extern __shared__ int s_pref[];  // [B + 1] prefix, then per wave [2][LIST] tile list
  __shared__ int s_wsum[MAX_HEADS_PER_WG];
  const int wg = blockIdx.x;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform over the wave: say so, so that page addresses stay scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int h = blockIdx.y * p.heads_per_wg + w;
  const int n16 = lane & 15, g4 = lane >> 4;
  const int G = p.G;

  // ---- inclusive prefix of tile counts over the batch (block-wide scan in chunks)
  int carry = 0;
  if (threadIdx.x == 0) s_pref[0] = 0;
  for (int base = 0; base < p.B; base += blockDim.x) {
    const int r = base + threadIdx.x;
    int v = r < p.B ? (sanitize_ctx(p, r) + 15) >> 4 : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(v, o, GP_WAVE);
      if (lane >= o) v += t;
    }
    if (lane == 63) s_wsum[w] = v;
    __syncthreads();
    int off = carry;
    for (int k = 0; k < w; ++k) off += s_wsum[k];
    int tot = 0;
    for (int k = 0; k < nw; ++k) tot += s_wsum[k];
    if (r < p.B) s_pref[r + 1] = off + v;
    carry += tot;
    __syncthreads();
  }
  const int U = s_pref[p.B];
  if (wg == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i <= p.B; i += blockDim.x) p.ws_pref[i] = s_pref[i];
  if (h >= p.H_kv) return;

  // ---- fused summary update (GrowPage Eq. 6 on the pre-RoPE queries): requests wg, wg + num_wg,
  // ... for this wave's KV head, independent of the tile ranges (empty requests included)
  if (p.q_pre) {
    const int GD = G * D;
    for (int r = wg; r < p.B; r += p.num_wg) {
      const int slot = p.slot_ids[r];
      if (slot < 0 || slot >= p.num_slots) continue;
      const bool fr = p.fresh[r] != 0;
      const size_t qb = ((size_t)r * p.H_q + (size_t)h * G) * D;
      const size_t sb = (size_t)slot * 2 * p.H_q * D + (size_t)h * G * D;
      for (int i = lane * 4; i < GD; i += 4 * GP_WAVE) {
        float x[4];
        gp::load_q4<KIND != KIND_F32>(p.q_pre, qb + i, x);
        gp::ema_update4(p.qstate + sb + i, p.qstate + sb + (size_t)p.H_q * D + i, x, fr, p.beta_s,
                        p.beta_l);
      }
    }
  }

  // this wave's tile lists in LDS, after the prefix: [LIST] page codes, then [LIST] tiles (a
  // mixed cache's first pass: bf16 tiles there, fp8 tiles in a second pair)
  int* lst_code = s_pref + pref_ints(p.B) + w * list_ints<KIND>();
  int* lst_tile = lst_code + LIST;
  int* lst_code2 = lst_tile + LIST;  // used by KIND_MIXED only
  int* lst_tile2 = lst_code2 + LIST;

  const int R = range_len(p, U);
  const long u0l = (long)wg * R;
  if (u0l >= U) return;
  const int u0 = (int)u0l, u1 = min(U, u0 + R);
  const int b = p.page_size;

  int u = u0;
  while (u < u1) {
    // request of unit u: the last r with s_pref[r] <= u (never an empty request)
    int lo = 0, hi = p.B;  // invariant: s_pref[lo] <= u < s_pref[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= u) lo = mid; else hi = mid;
    }
    const int r = lo;
    const int seg_end = min(u1, s_pref[r + 1]);
    const int ta = u - s_pref[r], tb = ta + (seg_end - u);
    const int ntiles = s_pref[r + 1] - s_pref[r];
    const int ctx = sanitize_ctx(p, r);
    u = seg_end;

    const int32_t* bt = p.block_tables + (size_t)r * p.max_pages;
    // query operand: head (lane % 16) of this KV head's group, zero rows past G
    const int hq0 = h * G;
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
    // half copy of the query for INT4 pages: step kk of lane (n16, g4) holds dimensions
    // g4 D/4 + 8 kk + (0, 4, 1, 5, 2, 6, 3, 7), the order the lane's key codes unpack in
    f16x8_t qh[KIND == KIND_INT4 ? D / 32 : 1];
    if constexpr (KIND == KIND_INT4) {
      const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + ((size_t)r * p.H_q + hq0 + n16) * D + (D / 4) * g4;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        const u32x4_t a = (n16 < G) ? *reinterpret_cast<const u32x4_t*>(qr + 8 * kk) : u32x4_t{0u, 0u, 0u, 0u};
        const float e0 = __uint_as_float(a.x << 16), e1 = __uint_as_float(a.x & 0xffff0000u);
        const float e2 = __uint_as_float(a.y << 16), e3 = __uint_as_float(a.y & 0xffff0000u);
        const float e4 = __uint_as_float(a.z << 16), e5 = __uint_as_float(a.z & 0xffff0000u);
        const float e6 = __uint_as_float(a.w << 16), e7 = __uint_as_float(a.w & 0xffff0000u);
        qh[kk] = f16x8_t{(_Float16)e0, (_Float16)e4, (_Float16)e1, (_Float16)e5,
                         (_Float16)e2, (_Float16)e6, (_Float16)e3, (_Float16)e7};
      }
    }

    WaveState<D> st;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) st.acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    for (int c0 = ta; c0 < tb; c0 += LIST) {
      // list of the tiles of [c0, c0 + LIST) this pass decodes, in order: page code and tile
      const int c1 = min(tb, c0 + LIST);
      int n = 0, n2 = 0;
      for (int k = 0; k < LIST; k += GP_WAVE) {
        const int t = c0 + k + lane;
        int code = -1;
        if (t < c1) {
          const int pg = bt[(t << 4) / b];
          code = (pg >= 0 && pg < p.num_pages) ? pg : -1;
          if constexpr (KIND == KIND_MIXED) {
            // bf16 and fp8 tiles; INT4 tiles belong to the second pass
            if (code >= 0) {
              const int tag = p.page_tag[pg];
              code = (tag == GP_TAG_FP8 || tag == GP_TAG_BF16) ? ((pg << 2) | tag) : -1;
            }
          } else if constexpr (KIND == KIND_INT4) {
            if (code >= 0) code = p.page_tag[pg] == GP_TAG_INT4 ? ((pg << 2) | GP_TAG_INT4) : -1;
          }
        }
        // fp8 tiles of a mixed cache go to the second list
        const bool second = KIND == KIND_MIXED && code >= 0 && (code & 3) == GP_TAG_FP8;
        const bool first = code >= 0 && !second;
        const uint64_t m = __builtin_amdgcn_ballot_w64(first);
        const uint64_t m2 = __builtin_amdgcn_ballot_w64(second);
        if (first) {
          const int at = n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          // a mixed cache's lists hold plain page ids (each list has one format)
          lst_code[at] = KIND == KIND_MIXED ? code >> 2 : code;
          lst_tile[at] = t;
        }
        if constexpr (KIND == KIND_MIXED) {
          if (second) {
            const int at = n2 + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m2 >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m2, 0u));
            lst_code2[at] = code >> 2;
            lst_tile2[at] = t;
          }
        }
        n += __builtin_popcountll(m);
        n2 += __builtin_popcountll(m2);
      }
      if constexpr (KIND == KIND_MIXED) {
        // bf16 tiles as a bf16 cache's (a scale of 1 changes no bit), then the fp8 tiles
        walk_tiles<D, KIND_BF16, RING>(p, lst_code, lst_tile, n, h, lane, ctx, qf, qh, st);
        walk_tiles<D, KIND_FP8, RING_FP8>(p, lst_code2, lst_tile2, n2, h, lane, ctx, qf, qh, st);
      } else if constexpr (KIND == KIND_INT4) {
        walk_tiles_int4<D>(p, lst_code, lst_tile, n, h, lane, ctx, qh, st);
      } else {
        walk_tiles<D, KIND, RING>(p, lst_code, lst_tile, n, h, lane, ctx, qf, qh, st);
      }
    }

    // ---- segment epilogue: final output rows, or a partial in slot j of this request
    float l_tot = st.l_run + __shfl_xor(st.l_run, 16, GP_WAVE);
    l_tot += __shfl_xor(l_tot, 32, GP_WAVE);
    float l_i[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) l_i[i] = __shfl(l_tot, 4 * g4 + i, GP_WAVE);
    // with two passes every segment leaves a partial, and the merge combines both passes
    const bool whole = ta == 0 && tb == ntiles && p.passes == 1;
    const int j = wg - s_pref[r] / R + p.pass * p.j_max;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 4 * g4 + i;
      if (head >= G) continue;
      const size_t row = (size_t)r * p.H_q + hq0 + head;
      if (whole) {
        const float inv = l_i[i] > 0.f ? 1.f / l_i[i] : 0.f;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) {
          const float o = st.acc[nb][i] * inv;
          if constexpr (KIND == KIND_F32)
            reinterpret_cast<float*>(p.out)[row * D + 16 * nb + n16] = o;
          else
            reinterpret_cast<uint16_t*>(p.out)[row * D + 16 * nb + n16] = (uint16_t)gp::f32_to_bf16_bits(o);
        }
      } else {
        float* wo = p.ws_o + (row * p.passes * p.j_max + j) * D;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) wo[16 * nb + n16] = st.acc[nb][i];
      }
    }
    if (g4 == 0 && n16 < G) {
      const size_t row = (size_t)r * p.H_q + hq0 + n16;
      if (whole) {
        if (p.lse) p.lse[row] = l_tot > 0.f ? (st.m_run + __log2f(l_tot)) * GP_LN2 : -INFINITY;
      } else {
        p.ws_ml[(row * p.passes * p.j_max + j) * 2 + 0] = st.m_run;
        p.ws_ml[(row * p.passes * p.j_max + j) * 2 + 1] = l_tot;
      }
    }
  }
}

// Merge of a request's partials (PASK App. B.5): o = sum_j e^{m_j - m} u_j / sum_j e^{m_j - m} l_j.
// One wave per output row; lane l holds partials l, l + 64, ... (J per pass, in slots
// pass * j_max + j), so the maximum, the denominator and the weights come from wave reductions
// and the partial outputs are fetched in one pass. With one pass, rows of requests that one
// workgroup finished are left as written; rows of empty requests get o = 0 and lse = -inf.
template <int D, int KIND>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeParams p) {
  const int lane = threadIdx.x & 63;
  // one output row per wave: its index is wave-uniform (scalar tests on the partial counts)
  const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (row >= (long)p.B * p.H_q) return;
  const int r = (int)(row / p.H_q);
  const int U = p.ws_pref[p.B];
  const int pa = p.ws_pref[r], pb = p.ws_pref[r + 1];
  // partials of each pass: the ranges of its stream-K width that overlap the request
  int Jp[2] = {0, 0};
  if (pb > pa) {
    for (int q = 0; q < p.passes; ++q) {
      const int R = range_len(p.num_wg_pass[q], p.r_min, U);
      Jp[q] = (pb - 1) / R - pa / R + 1;
    }
  }
  if (Jp[0] == 1 && p.passes == 1) return;
  // J <= j_max <= J_CAP_MAX + 1 = 128 per pass: at most 4 partials per lane
  const int J0 = Jp[0], NP = Jp[0] + Jp[1];
  const int SL = p.passes * p.j_max;  // slots per row
  auto slot = [&](int k) { return k < J0 ? k : p.j_max + (k - J0); };  // k < NP
  const float* ml = p.ws_ml + row * SL * 2;
  const float* wo = p.ws_o + row * SL * D;
  constexpr int PER = D / 64;
  constexpr int BATCH = 8;  // partial rows fetched before any is used
  float x[BATCH][PER];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e)
        x[u][e] = k0 + u < NP ? wo[(size_t)slot(k0 + u) * D + lane + 64 * e] : 0.f;
  };
  // the first batch of partial rows goes out with the (max, sum) loads: they depend only on the
  // partial count, so a row with at most BATCH partials waits for one round trip, not two
  fetch(0);
  float mk[4], lk[4];
  float mloc = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = lane + 64 * q;
    mk[q] = k < NP ? ml[2 * slot(k)] : -INFINITY;
    lk[q] = k < NP ? ml[2 * slot(k) + 1] : 0.f;
    mloc = fmaxf(mloc, mk[q]);
  }
  const float m = gp::wave_max(mloc);
  float wk[4], dsum = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    wk[q] = gp::safe_exp2_diff(mk[q], m);
    dsum += wk[q] * lk[q];
  }
  const float den = gp::wave_sum(dsum);
  const float inv = den > 0.f ? 1.f / den : 0.f;
  float num[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) num[e] = 0.f;
  for (int k0 = 0; k0 < NP; k0 += BATCH) {
    if (k0 > 0) fetch(k0);
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int k = k0 + u;
      float wt = 0.f;
      if (k < NP) {
        const int q = k >> 6;
        const float wq = q == 0 ? wk[0] : q == 1 ? wk[1] : q == 2 ? wk[2] : wk[3];
        wt = __shfl(wq, k & 63, GP_WAVE);
      }
#pragma unroll
      for (int e = 0; e < PER; ++e) num[e] += wt > 0.f ? wt * x[u][e] : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const float o = num[e] * inv;
    const size_t at = row * D + lane + 64 * e;
    if constexpr (KIND == KIND_F32)
      reinterpret_cast<float*>(p.out)[at] = o;
    else
      reinterpret_cast<uint16_t*>(p.out)[at] = (uint16_t)gp::f32_to_bf16_bits(o);
  }
  if (lane == 0 && p.lse) p.lse[row] = den > 0.f ? (m + __log2f(den)) * GP_LN2 : -INFINITY;
}

struct Plan {
  int r_min, j_max;
};

// KV heads per workgroup: the largest divisor of H_kv up to `cap`, so that every wave of every
// workgroup has a head (12 KV heads: two workgroups of 6 rather than 8 + 4 and 4 idle waves).
int heads_per_workgroup(int H_kv, int cap) {
  for (int k = std::min(H_kv, cap); k > 1; --k)
    if (H_kv % k == 0) return k;
  return 1;
}

// Ranges hold at least r_min tiles, so one request is spread over at most j_max workgroups.
Plan plan_for(int B, int max_context) {
  const int max_tiles = (max_context + 15) / 16;
  // a batch of many requests fills the device with few splits each; a small batch of long
  // requests needs more of them (the workspace grows with B * j_max either way)
  const int j_cap = std::min(J_CAP_MAX, std::max(16, 1024 / std::max(B, 1)));
  Plan pl;
  pl.r_min = std::max(8, (max_tiles + j_cap - 1) / j_cap);
  pl.j_max = (max_tiles + pl.r_min - 1) / pl.r_min + 1;
  return pl;
}

// Workgroups of the streaming kernel that fit on the device at once. Memoised per device and
// instantiation: each entry is one 64-bit atomic holding the query (block size and LDS bytes)
// in its high half and the answer in its low half, so a reader never pairs one query with
// another's answer. Only host-side device properties are cached.
template <int D, int KIND, int RING>
int resident_workgroups(int threads, size_t lds) {
  static std::atomic<uint64_t> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const uint32_t key = (uint32_t)threads << 16 | (uint32_t)std::min<size_t>(lds, 65535);
  if (dev < 64) {
    const uint64_t e = cache[dev].load(std::memory_order_relaxed);
    if ((uint32_t)(e >> 32) == key && (uint32_t)e > 0) return (int)(uint32_t)e;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_streamk_kernel<D, KIND, RING>, threads,
                                                   lds) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int v = cus * per_cu;
  if (dev < 64) cache[dev].store((uint64_t)key << 32 | (uint32_t)v, std::memory_order_relaxed);
  return v;
}

// compute units of the current device (memoised per device; host-side property only)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int D, int KIND, int RING>
int launch_decode_ring(DecodeParams p, int max_workgroups, hipStream_t stream, uint32_t tags) {
  const int hg = (p.H_kv + p.heads_per_wg - 1) / p.heads_per_wg;
  const int threads = p.heads_per_wg * GP_WAVE;
  const size_t lds = ((size_t)pref_ints(p.B) + (size_t)p.heads_per_wg * list_ints<KIND>()) * sizeof(int);
  // a mixed cache decodes in two passes over the same ranges (the bf16 / fp8 tiles, then the
  // INT4 tiles with a deeper ring); both must cut the batch identically. A pass whose page tags
  // the caller declares absent is not launched (tags == 0: unknown, both run); with no INT4 pass
  // left the first runs alone, and with no first pass the INT4 pass runs alone as pass 0.
  bool run_first = true, run_int4 = KIND == KIND_MIXED;
  if (KIND == KIND_MIXED && tags != 0) {
    run_int4 = (tags & (1u << GP_TAG_INT4)) != 0;
    run_first = (tags & ((1u << GP_TAG_BF16) | (1u << GP_TAG_FP8))) != 0 || !run_int4;
  }
  p.passes = (run_first ? 1 : 0) + (run_int4 ? 1 : 0);
  int total = resident_workgroups<D, KIND, RING>(threads, lds);
  if (max_workgroups > 0) total = std::min(total, max_workgroups);
  p.num_wg = std::max(1, total / hg);
  p.pass = 0;
  // the INT4 pass has its own geometry: smaller workgroups, so that more waves hide latency
  const int hpw1 = heads_per_workgroup(p.H_kv, INT4_HEADS_PER_WG);
  const int hg1 = (p.H_kv + hpw1 - 1) / hpw1;
  int total1 = 0;
  const size_t lds1 = ((size_t)pref_ints(p.B) + (size_t)hpw1 * list_ints<KIND_INT4>()) * sizeof(int);
  if (run_int4) {
    total1 = resident_workgroups<D, KIND_INT4, RING_INT4>(hpw1 * GP_WAVE, lds1);
    if (max_workgroups > 0) total1 = std::min(total1, max_workgroups * (p.heads_per_wg / hpw1));
  }
  const int width1 = std::max(1, total1 / hg1);
  p.num_wg_pass[0] = run_first ? p.num_wg : width1;
  p.num_wg_pass[1] = run_first && run_int4 ? width1 : 1;
  if (run_first) {
    hipLaunchKernelGGL((decode_streamk_kernel<D, KIND, RING>), dim3(p.num_wg, hg), dim3(threads), lds,
                       stream, p);
    GP_CHECK_LAUNCH();
  }
  if (run_int4) {
    DecodeParams p1 = p;
    p1.pass = run_first ? 1 : 0;
    if (run_first) p1.q_pre = nullptr;  // the summary update ran in the first pass
    p1.heads_per_wg = hpw1;
    p1.num_wg = width1;
    hipLaunchKernelGGL((decode_streamk_kernel<D, KIND_INT4, RING_INT4>), dim3(p1.num_wg, hg1),
                       dim3(hpw1 * GP_WAVE), lds1, stream, p1);
    GP_CHECK_LAUNCH();
  }
  const long rows = (long)p.B * p.H_q;
  hipLaunchKernelGGL((decode_merge_kernel<D, KIND>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     stream, p);
  GP_CHECK_LAUNCH();
  return GP_OK;
}

// Ring depth of the call: one tile in flight per wave for a capped bf16 / fp32 decode (one that
// shares the GPU), two otherwise. Mixed caches always use two. An uncapped call over eight-head
// workgroups of 128-dimensional heads (32 KB of K and V per tile and workgroup) also keeps one
// tile per wave, with one workgroup per compute unit: that streams faster than two tiles per
// wave with the same grid (Qwen3-8B-shaped batch 0.422 -> 0.413 ms) or than two workgroups per
// compute unit (0.432 ms). Smaller tiles need the deeper ring to keep enough bytes in flight.
template <int D, int KIND>
int launch_decode(DecodeParams p, int max_workgroups, hipStream_t stream, uint32_t tags) {
  if constexpr (KIND == KIND_BF16 || KIND == KIND_F32) {
    if (max_workgroups > 0) return launch_decode_ring<D, KIND, RING_SHARED>(p, max_workgroups, stream, 0);
    if (D == 128 && p.heads_per_wg == MAX_HEADS_PER_WG) {
      const int hg = (p.H_kv + p.heads_per_wg - 1) / p.heads_per_wg;
      return launch_decode_ring<D, KIND, RING_SHARED>(p, device_cus() * hg, stream, 0);
    }
  }
  return launch_decode_ring<D, KIND, RING_FULL>(p, max_workgroups, stream, tags);
}

// Bytes of the decode workspace when `passes` passes leave partials (a mixed cache decodes its
// INT4 tiles in a pass of their own): the prefix of tile counts, 256-byte aligned, then every
// output row's partial outputs and partial (max, sum) pairs.
size_t decode_ws_bytes(int B, int H_q, int head_dim, int max_context, int passes) {
  const Plan pl = plan_for(B, max_context);
  const size_t partials = (size_t)B * H_q * passes * pl.j_max * (head_dim + 2) * sizeof(float);
  const size_t pref = ((size_t)(B + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
  return pref + partials;
}

// Scratch of gp_paged_decode_attn_noalloc: a static device array, one copy on every device the
// library runs on, held until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): it takes the device address that
// hipGetSymbolAddress returns for the current device, looked up on the first call on that device.
static __device__ __align__(256) unsigned char scratch[GP_NOALLOC_SCRATCH_BYTES];

int scratch_on_current_device(void** out) {
  static std::atomic<void*> ptrs[64];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GP_ERR_HIP;
  if (dev >= 64) return GP_ERR_UNSUPPORTED;
  void* ptr = ptrs[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GP_ERR_HIP;
    ptrs[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return GP_OK;
}

}  // namespace

extern "C" size_t gp_paged_decode_attn_workspace_size(int B, int H_q, int H_kv, int head_dim,
                                                      int page_size, int max_context) {
  (void)page_size;
  (void)H_kv;
  if (B <= 0 || H_q <= 0 || head_dim <= 0 || max_context < 0) return 0;
  return decode_ws_bytes(B, H_q, head_dim, max_context, 2);
}

namespace {

// static_scratch: take the workspace from the library's static scratch on the current device
// (workspace / workspace_bytes are ignored), laid out for the passes this call needs.
int decode_impl(const void* q, int q_dtype, int B, int H_q, const gp_kv_cache* kv,
                const int32_t* block_tables, int max_pages, const int32_t* context_lens,
                int max_context, float sm_scale, void* out, float* lse,
                const gp_summary_update* upd, int max_workgroups, void* workspace,
                size_t workspace_bytes, void* stream, bool static_scratch = false) {
  if (B < 0 || H_q <= 0 || !kv || max_pages <= 0 || max_context < 0) return GP_ERR_INVALID;
  if (max_workgroups < 0) return GP_ERR_INVALID;
  if (upd && (!upd->q_pre || !upd->slot_ids || !upd->fresh || !upd->qstate || upd->num_slots <= 0))
    return GP_ERR_INVALID;
  if (B == 0) return GP_OK;
  if (!q || !out || !block_tables || !context_lens || !kv->k || !kv->v) return GP_ERR_INVALID;
  const int H_kv = kv->num_kv_heads, D = kv->head_dim, b = kv->page_size;
  if (H_kv <= 0 || H_q % H_kv != 0 || kv->num_pages <= 0) return GP_ERR_INVALID;
  if (b < 16 || b > 256 || b % 16 != 0) return GP_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return GP_ERR_UNSUPPORTED;
  const int G = H_q / H_kv;
  if (G > 16) return GP_ERR_UNSUPPORTED;
  if (B > MAX_BATCH) return GP_ERR_UNSUPPORTED;
  if (q_dtype != kv->dtype || (q_dtype != GP_F32 && q_dtype != GP_BF16)) return GP_ERR_INVALID;
  const bool mixed = kv->page_tag != nullptr;
  if (mixed && (q_dtype != GP_BF16 || !kv->k8 || !kv->v8 || !kv->k_scale || !kv->v_scale ||
                !kv->k4 || !kv->v4 || !kv->k4_scale || !kv->v4_scale))
    return GP_ERR_INVALID;
  if ((long)max_context > (long)max_pages * b) return GP_ERR_INVALID;
  if ((long)kv->num_pages * H_kv * b > (1L << 40)) return GP_ERR_INVALID;
  if ((long)kv->num_pages * 4 > (long)INT32_MAX) return GP_ERR_UNSUPPORTED;  // tag packing
  if ((long)B * ((max_context + 15) / 16) > (long)INT32_MAX / 2) return GP_ERR_UNSUPPORTED;

  const int passes = mixed ? 2 : 1;
  if (static_scratch) {
    if (decode_ws_bytes(B, H_q, D, max_context, passes) > GP_NOALLOC_SCRATCH_BYTES)
      return GP_ERR_SCRATCH;
    const int st = scratch_on_current_device(&workspace);
    if (st != GP_OK) return st;
  } else {
    const size_t need = gp_paged_decode_attn_workspace_size(B, H_q, H_kv, D, b, max_context);
    if (!workspace || workspace_bytes < need) return GP_ERR_WORKSPACE;
  }
  const Plan pl = plan_for(B, max_context);

  DecodeParams p{};
  p.q = q;
  p.k = kv->k;
  p.v = kv->v;
  p.k8 = static_cast<const uint8_t*>(kv->k8);
  p.v8 = static_cast<const uint8_t*>(kv->v8);
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  p.k4 = static_cast<const uint8_t*>(kv->k4);
  p.v4 = static_cast<const uint8_t*>(kv->v4);
  p.k4_scale = kv->k4_scale;
  p.v4_scale = kv->v4_scale;
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
  p.heads_per_wg = heads_per_workgroup(H_kv, MAX_HEADS_PER_WG);
  p.r_min = pl.r_min;
  p.j_max = pl.j_max;
  p.scale_log2 = sm_scale * GP_LOG2E;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.ws_pref = reinterpret_cast<int32_t*>(ws);
  p.ws_o = reinterpret_cast<float*>(ws + (((size_t)(B + 1) * sizeof(int32_t) + 255) & ~(size_t)255));
  p.ws_ml = p.ws_o + (size_t)B * H_q * passes * pl.j_max * D;
  if (upd) {
    p.q_pre = upd->q_pre;
    p.slot_ids = upd->slot_ids;
    p.fresh = upd->fresh;
    p.qstate = upd->qstate;
    p.num_slots = upd->num_slots;
    p.beta_s = upd->beta_s;
    p.beta_l = upd->beta_l;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mw = max_workgroups;
  const uint32_t tags = mixed ? kv->tags_present : 0u;
  if (mixed) return D == 64 ? launch_decode<64, KIND_MIXED>(p, mw, s, tags) : launch_decode<128, KIND_MIXED>(p, mw, s, tags);
  if (q_dtype == GP_BF16) return D == 64 ? launch_decode<64, KIND_BF16>(p, mw, s, 0) : launch_decode<128, KIND_BF16>(p, mw, s, 0);
  return D == 64 ? launch_decode<64, KIND_F32>(p, mw, s, 0) : launch_decode<128, KIND_F32>(p, mw, s, 0);
}

}  // namespace

extern "C" int gp_paged_decode_attn(const void* q, int q_dtype, int B, int H_q,
                                    const gp_kv_cache* kv, const int32_t* block_tables,
                                    int max_pages, const int32_t* context_lens, int max_context,
                                    float sm_scale, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_dtype, B, H_q, kv, block_tables, max_pages, context_lens, max_context,
                     sm_scale, out, lse, nullptr, 0, workspace, workspace_bytes, stream);
}

extern "C" int gp_paged_decode_attn_ex(const void* q, int q_dtype, int B, int H_q,
                                       const gp_kv_cache* kv, const int32_t* block_tables,
                                       int max_pages, const int32_t* context_lens,
                                       int max_context, float sm_scale, void* out, float* lse,
                                       const gp_summary_update* summaries, int max_workgroups,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, q_dtype, B, H_q, kv, block_tables, max_pages, context_lens, max_context,
                     sm_scale, out, lse, summaries, max_workgroups, workspace, workspace_bytes,
                     stream);
}

extern "C" int gp_paged_decode_attn_noalloc(const void* q, int q_dtype, int B, int H_q,
                                            const gp_kv_cache* kv, const int32_t* block_tables,
                                            int max_pages, const int32_t* context_lens,
                                            int max_context, float sm_scale, void* out, float* lse,
                                            const gp_summary_update* summaries, int max_workgroups,
                                            void* stream) {
  return decode_impl(q, q_dtype, B, H_q, kv, block_tables, max_pages, context_lens, max_context,
                     sm_scale, out, lse, summaries, max_workgroups, nullptr, 0, stream, true);
}
