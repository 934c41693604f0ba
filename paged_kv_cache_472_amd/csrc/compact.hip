// Compress-or-grow at a page boundary for gfx950 (GrowPage Sec. 3.2 Eq. 8 decision, Sec. 3.3
// Eq. 9-10 selection and Compress & Hold / Grow by One Page, Sec. 4.2 and App. E.2 free-page pool,
// fallback and prefix-safe compaction, App. H.1 policies).
//
// Launches:
//   1. decide_alloc (one wave): requests in req_idx order. Decision from the exact comparison of
//      sum_h (K^S_h - K^L_h) / (H |C|) with tau; Grow pops the LIFO free stack; compression pops
//      one private page per shared page it must write (wave-parallel ballot ranks, ascending
//      logical order); released references are applied after every pop of the call.
//   2. select (per request x KV head, 1024 threads): s = max(a^S, a^L) held in registers, 32
//      consecutive candidates per thread so each thread ranks whole pages for the k_loc quota;
//      the E <= page_size evicted tokens are found by E rounds of a block-wide minimum over the
//      unique keys (s, ~index), which realises the (s desc, index asc) order exactly.
//   3. snapshot: compaction is a left shift by at most E slots, so a chunk of destination pages
//      only reads its own pages plus the first page of the next chunk; that page is saved first.
//   4. compact (per chunk x KV head x request): read all sources (keys row-wise from HBM, values
//      through LDS), barrier, write the chunk's destination pages.
#include "common.h"

namespace {

constexpr int MODE_NONE = 0;      // grow / no pages: kept_idx = -1 over |C|
constexpr int MODE_IDENTITY = 1;  // compress with nothing to evict: kept_idx = 0..|C|-1
constexpr int MODE_COMPACT = 2;
constexpr int SEL_THREADS = 1024;
constexpr int SEL_VPT = 32;
constexpr int MAX_EVICT = 32;
constexpr int CP_THREADS = 256;
constexpr int CP_LDS_BYTES = 48 * 1024;

struct Info {
  int r, mode, P, ctx_old, n, K_t, R_n, E, ctx_new, n_dest, first_repl, pad;
};

struct CParams {
  const int32_t* req_idx;
  const float* a_short;
  const float* a_long;
  const int32_t* ws_counts;
  const int32_t* n_cand;
  const int32_t* policies;
  uint8_t* k;
  uint8_t* v;
  int32_t* block_tables;
  int32_t* n_pages;
  int32_t* context_lens;
  int32_t* refcount;
  int32_t* free_stack;
  int32_t* free_top;
  int32_t* decision;
  int32_t* kept_idx;
  Info* info;         // [R]
  int32_t* old_bt;    // [R, max_pages]
  int32_t* rel;       // [R * max_pages]
  int32_t* ev;        // [R, H_kv, MAX_EVICT]
  int32_t* dp0;       // [R, H_kv]
  uint8_t* snap;      // [R, H_kv, max_chunks, 2, page bytes]
  int R, B, H_kv, D, page_size, num_pages, max_pages, C_max, k_loc, policy, es;
  int chunk_pages, max_chunks;
  double tau;
};

// grow iff D / (H n) > tau, decided exactly (D integer, tau a double)
__device__ bool trend_exceeds(long long Dsum, long long HN, double tau) {
  if (tau == 0.0) return Dsum > 0;
  int E;
  const double f = frexp(tau, &E);                         // tau = f 2^E, 0.5 <= |f| < 1
  const long long mant = (long long)ldexp(f, 53);          // tau = mant 2^(E-53) exactly
  if (E > 40) return tau < 0.0;                            // |tau H n| far beyond |D|
  const __int128 prod = (__int128)mant * (__int128)HN;     // tau H n = prod 2^(E-53)
  const int s = 53 - E;                                    // s >= 13
  __int128 fl;
  if (s >= 120) fl = prod < 0 ? (__int128)-1 : (__int128)0;
  else fl = prod >> s;                                     // floor(tau H n)
  return (__int128)Dsum > fl;                              // integer D > x  <=>  D > floor(x)
}

__global__ __launch_bounds__(64) void decide_alloc_kernel(CParams P) {
  const int lane = threadIdx.x;
  const int b = P.page_size;
  int top = *P.free_top;
  if (top < 0 || top > P.num_pages) top = 0;
  int nrel = 0;
  for (int i = 0; i < P.R; ++i) {
    Info inf = {};
    inf.mode = MODE_NONE;
    const int nc = P.n_cand[i];
    inf.n = (nc > 0 && nc <= P.C_max) ? nc : 0;
    int dec = GP_DECISION_NO_PAGES;
    const int r = P.req_idx[i];
    inf.r = r;
    bool ok = r >= 0 && r < P.B && nc >= 0 && nc <= P.C_max;
    int Pn = 0, ctx = 0;
    if (ok) {
      Pn = P.n_pages[r];
      ctx = P.context_lens[r];
      ok = Pn >= 1 && Pn <= P.max_pages && ctx >= 0 && (long)ctx <= (long)Pn * b;
    }
    int n = 0;
    if (ok) {
      n = ctx == 0 ? 0 : ((ctx + b - 1) / b - 1) * b;
      ok = n == nc;
    }
    // sum over KV heads of K^S - K^L
    long long dsum = 0;
    bool bad_ws = false;
    if (ok) {
      for (int h = lane; h < P.H_kv; h += 64) {
        const int ks = P.ws_counts[((size_t)i * P.H_kv + h) * 2 + 0];
        const int kl = P.ws_counts[((size_t)i * P.H_kv + h) * 2 + 1];
        if (ks < 0 || kl < 0) bad_ws = true;
        dsum += (long long)ks - kl;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) dsum += __shfl_xor(dsum, o, GP_WAVE);
      bad_ws = __any(bad_ws);
      if (n > 0 && bad_ws) ok = false;
    }
    if (!ok) {
      if (lane == 0) {
        P.decision[i] = GP_DECISION_NO_PAGES;
        P.info[i] = inf;
      }
      continue;
    }
    const int pol = P.policies ? P.policies[i] : P.policy;
    bool want_grow;
    if (pol == GP_POLICY_FORCE_COMPRESS) want_grow = false;
    else if (pol == GP_POLICY_FORCE_GROW || n == 0) want_grow = true;
    else {
      const bool g = trend_exceeds(dsum, (long long)P.H_kv * n, P.tau);
      want_grow = (pol == GP_POLICY_INVERSE) ? !g : g;
    }
    int code = GP_DECISION_COMPRESS;
    bool done = false;
    if (want_grow) {
      if (top > 0 && Pn < P.max_pages) {
        if (lane == 0) {
          const int pg = P.free_stack[top - 1];
          P.free_stack[top - 1] = -1;
          P.block_tables[(size_t)r * P.max_pages + Pn] = pg;
          P.n_pages[r] = Pn + 1;
          if (pg >= 0 && pg < P.num_pages) P.refcount[pg] = 1;
        }
        --top;
        dec = GP_DECISION_GROW;
        done = true;
      } else if (n == 0) {
        dec = GP_DECISION_NO_PAGES;
        done = true;
      } else {
        code = GP_DECISION_GROW_FALLBACK_COMPRESS;
      }
    }
    if (!done) {
      const int R_n = ctx - n;
      const int K_t = min(n, max(0, (Pn - 1) * b - R_n));
      const int E = n - K_t;
      inf.P = Pn;
      inf.ctx_old = ctx;
      inf.K_t = K_t;
      inf.R_n = R_n;
      inf.E = E;
      if (E == 0) {
        inf.mode = MODE_IDENTITY;
        dec = code;
      } else if (E > MAX_EVICT) {
        dec = GP_DECISION_NO_PAGES;  // unreachable for page sizes <= 32 (E <= page_size)
      } else {
        const int ctx_new = K_t + R_n;
        const int n_dest = (ctx_new + b - 1) / b;
        int32_t* row = P.block_tables + (size_t)r * P.max_pages;
        int cnt = 0;
        bool bad = false;
        // every page the compaction may read (all Pn) must be a valid id; the first n_dest
        // are written, so the shared ones among them need a replacement
        for (int j0 = 0; j0 < Pn; j0 += 64) {
          const int j = j0 + lane;
          bool sh = false;
          if (j < Pn) {
            const int pg = row[j];
            if (pg < 0 || pg >= P.num_pages) bad = true;
            else sh = j < n_dest && P.refcount[pg] > 1;
          }
          cnt += __popcll(__ballot(sh));
        }
        bad = __any(bad);
        if (bad || cnt > top) {
          dec = GP_DECISION_NO_PAGES;
        } else {
          for (int j = lane; j < Pn; j += 64) P.old_bt[(size_t)i * P.max_pages + j] = row[j];
          int base = 0;
          int first = n_dest;
          for (int j0 = 0; j0 < n_dest; j0 += 64) {
            const int j = j0 + lane;
            bool sh = false;
            int pg = -1;
            if (j < n_dest) {
              pg = row[j];
              sh = P.refcount[pg] > 1;
            }
            const unsigned long long m = __ballot(sh);
            if (m && first == n_dest) first = j0 + __ffsll((long long)m) - 1;
            const int rank = base + __popcll(m & ((1ull << lane) - 1ull));
            if (sh) {
              const int np = P.free_stack[top - 1 - rank];
              P.free_stack[top - 1 - rank] = -1;
              P.rel[nrel + rank] = pg;
              row[j] = np;
              if (np >= 0 && np < P.num_pages) P.refcount[np] = 1;
            }
            base += __popcll(m);
          }
          top -= cnt;
          nrel += cnt;
          if (lane == 0) P.context_lens[r] = ctx_new;
          inf.mode = MODE_COMPACT;
          inf.ctx_new = ctx_new;
          inf.n_dest = n_dest;
          inf.first_repl = first;
          dec = code;
        }
      }
    }
    if (lane == 0) {
      P.decision[i] = dec;
      P.info[i] = inf;
    }
  }
  __threadfence();
  __syncthreads();
  if (lane == 0) {
    for (int k = 0; k < nrel; ++k) {
      const int pg = P.rel[k];
      const int rc = P.refcount[pg] - 1;
      P.refcount[pg] = rc;
      if (rc == 0 && top < P.num_pages) P.free_stack[top++] = pg;
    }
    *P.free_top = top;
  }
}

__device__ __forceinline__ unsigned long long block_min_u64(unsigned long long v, unsigned long long* scratch) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long t = __shfl_xor(v, o, GP_WAVE);
    v = t < v ? t : v;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) scratch[w] = v;
  __syncthreads();
  unsigned long long m = ~0ull;
  for (int k = 0; k < SEL_THREADS / GP_WAVE; ++k) m = scratch[k] < m ? scratch[k] : m;
  return m;
}

template <int PB>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(CParams P) {
  const int h = blockIdx.x, i = blockIdx.y;
  const Info inf = P.info[i];
  const int n = inf.n;
  int32_t* out = P.kept_idx + ((size_t)i * P.H_kv + h) * P.C_max;
  if (inf.mode != MODE_COMPACT) {
    for (int t = threadIdx.x; t < n; t += SEL_THREADS) out[t] = inf.mode == MODE_IDENTITY ? t : -1;
    return;
  }
  constexpr int b = PB;
  const int K_t = inf.K_t, E = inf.E;
  const int t0 = threadIdx.x * SEL_VPT;
  const float* as = P.a_short + ((size_t)i * P.H_kv + h) * P.C_max;
  const float* al = P.a_long + ((size_t)i * P.H_kv + h) * P.C_max;
  uint32_t s[SEL_VPT];
#pragma unroll
  for (int j = 0; j < SEL_VPT; j += 4) {
    if (t0 + j < n) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(as + t0 + j);
      const f32x4_t y = *reinterpret_cast<const f32x4_t*>(al + t0 + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[j + e] = max(__float_as_uint(x[e]) & 0x7fffffffu, __float_as_uint(y[e]) & 0x7fffffffu);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) s[j + e] = 0u;
    }
  }
  const int kloc = min(P.k_loc, b);
  const long n_loc = (long)(n / b) * kloc;
  const bool pool_all = n_loc >= K_t;
  unsigned long long key[SEL_VPT];
#pragma unroll
  for (int j = 0; j < SEL_VPT; ++j) {
    const int t = t0 + j;
    bool cand = t < n;
    if (cand && !pool_all) {
      // rank of t inside its page under (s desc, index asc); pages never straddle threads
      const int pbase = (j / b) * b;
      int rank = 0;
#pragma unroll
      for (int u = 0; u < b; ++u) {
        const int ju = pbase + u;
        const bool better = s[ju] > s[j] || (s[ju] == s[j] && ju < j);
        rank += better ? 1 : 0;
      }
      cand = rank >= kloc;
    }
    key[j] = cand ? (((unsigned long long)s[j] << 32) | (0xffffffffu - (uint32_t)t)) : ~0ull;
  }
  __shared__ unsigned long long scratch[SEL_THREADS / GP_WAVE];
  __shared__ int s_ev[MAX_EVICT], s_sorted[MAX_EVICT];
  unsigned long long prev = 0;
  for (int e = 0; e < E; ++e) {
    unsigned long long m = ~0ull;
#pragma unroll
    for (int j = 0; j < SEL_VPT; ++j) {
      const bool ok = (e == 0) || key[j] > prev;
      if (ok && key[j] < m) m = key[j];
    }
    m = block_min_u64(m, scratch);
    prev = m;
    if (threadIdx.x == 0) s_ev[e] = (int)(0xffffffffu - (uint32_t)(m & 0xffffffffu));
  }
  __syncthreads();
  if (threadIdx.x < E) {
    const int v = s_ev[threadIdx.x];
    int rank = 0;
    for (int e = 0; e < E; ++e) rank += s_ev[e] < v ? 1 : 0;
    s_sorted[rank] = v;
  }
  __syncthreads();
  if (threadIdx.x < E) {
    P.ev[((size_t)i * P.H_kv + h) * MAX_EVICT + threadIdx.x] = s_sorted[threadIdx.x];
    out[K_t + threadIdx.x] = -1;
  }
  if (threadIdx.x == 0) P.dp0[(size_t)i * P.H_kv + h] = min(s_sorted[0] / b, inf.first_repl);
  // kept tokens in ascending order: token t goes to t - #(evicted < t)
#pragma unroll
  for (int j = 0; j < SEL_VPT; ++j) {
    const int t = t0 + j;
    if (t >= n) continue;
    int before = 0;
    bool evicted = false;
    for (int e = 0; e < E; ++e) {
      before += s_sorted[e] < t ? 1 : 0;
      evicted |= s_sorted[e] == t;
    }
    if (!evicted) out[t - before] = t;
  }
}

// page bytes of one KV head: keys [b][D], values [D][b]
__device__ __forceinline__ size_t page_bytes(const CParams& P) { return (size_t)P.page_size * P.D * P.es; }
__device__ __forceinline__ size_t pool_off(const CParams& P, int pg, int h) {
  return ((size_t)pg * P.H_kv + h) * page_bytes(P);
}
__device__ __forceinline__ uint8_t* snap_ptr(const CParams& P, int i, int h, int c, int which) {
  return P.snap + ((((size_t)i * P.H_kv + h) * P.max_chunks + c) * 2 + which) * page_bytes(P);
}
// does the chunk that ends at logical page lp read lp from the snapshot?
__device__ __forceinline__ bool from_snapshot(const CParams& P, int lp, int dp0, int n_dest) {
  return (lp % P.chunk_pages) == 0 && lp > dp0 && lp < n_dest;
}

__global__ __launch_bounds__(CP_THREADS) void snapshot_kernel(CParams P) {
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Info inf = P.info[i];
  if (inf.mode != MODE_COMPACT || c == 0) return;
  const int lp = c * P.chunk_pages;
  const int dp0 = P.dp0[(size_t)i * P.H_kv + h];
  if (!from_snapshot(P, lp, dp0, inf.n_dest)) return;
  const int pg = P.old_bt[(size_t)i * P.max_pages + lp];
  const size_t nb = page_bytes(P);
  const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(P.k + pool_off(P, pg, h));
  const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(P.v + pool_off(P, pg, h));
  u32x4_t* kd = reinterpret_cast<u32x4_t*>(snap_ptr(P, i, h, c, 0));
  u32x4_t* vd = reinterpret_cast<u32x4_t*>(snap_ptr(P, i, h, c, 1));
  for (size_t q = threadIdx.x; q < nb / 16; q += CP_THREADS) {
    kd[q] = ks[q];
    vd[q] = vs[q];
  }
}

// source position of destination slot j: the j-th kept token, then the recent tokens
__device__ __forceinline__ int src_of(int j, const int* ev, int E) {
  int k = 0;
  while (k < E && ev[k] <= j + k) ++k;
  return j + k;
}

template <int ITEMS>
__global__ __launch_bounds__(CP_THREADS) void compact_kernel(CParams P) {
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Info inf = P.info[i];
  if (inf.mode != MODE_COMPACT) return;
  const int L = P.chunk_pages, b = P.page_size, D = P.D, es = P.es;
  const int dp0 = P.dp0[(size_t)i * P.H_kv + h];
  const int dp_lo = max(dp0, c * L), dp_hi = min((c + 1) * L, inf.n_dest);
  if (dp_lo >= dp_hi) return;
  __shared__ int s_ev[MAX_EVICT];
  extern __shared__ __align__(16) uint8_t s_v[];  // value pages [dp_lo .. dp_hi] of this head
  const int E = inf.E;
  if (threadIdx.x < E) s_ev[threadIdx.x] = P.ev[((size_t)i * P.H_kv + h) * MAX_EVICT + threadIdx.x];
  const int32_t* obt = P.old_bt + (size_t)i * P.max_pages;
  const int32_t* nbt = P.block_tables + (size_t)inf.r * P.max_pages;
  const size_t pb = page_bytes(P);
  const int q_per_page = (int)(pb / 16);
  // stage the source value pages through LDS (coalesced 16-byte loads)
  const int nsrc = dp_hi - dp_lo + 1;
  for (int q = threadIdx.x; q < nsrc * q_per_page; q += CP_THREADS) {
    const int sp = q / q_per_page, qq = q % q_per_page;
    const int lp = dp_lo + sp;
    u32x4_t val = u32x4_t{0u, 0u, 0u, 0u};
    if (lp < inf.P) {
      const uint8_t* src = from_snapshot(P, lp, dp0, inf.n_dest) ? snap_ptr(P, i, h, lp / L, 1)
                                                                  : P.v + pool_off(P, obt[lp], h);
      val = reinterpret_cast<const u32x4_t*>(src)[qq];
    }
    reinterpret_cast<u32x4_t*>(s_v)[q] = val;
  }
  __syncthreads();
  // read phase: keys (16-byte pieces of rows) and value pieces (16 bytes of a value row)
  const int kq_row = D * es / 16;           // 16-byte pieces per key row
  const int n_items_k = (dp_hi - dp_lo) * b * kq_row;
  const int vq_row = b * es / 16;           // 16-byte pieces per value row of a page
  const int n_items_v = (dp_hi - dp_lo) * D * vq_row;
  u32x4_t kreg[ITEMS], vreg[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int q = threadIdx.x + it * CP_THREADS;
    if (q < n_items_k) {
      const int slot_g = q / kq_row, piece = q % kq_row;
      const int j = dp_lo * b + slot_g;
      const int sidx = src_of(j, s_ev, E);
      const int lp = sidx / b, so = sidx % b;
      const uint8_t* base = from_snapshot(P, lp, dp0, inf.n_dest) ? snap_ptr(P, i, h, lp / L, 0)
                                                                   : P.k + pool_off(P, obt[lp], h);
      kreg[it] = reinterpret_cast<const u32x4_t*>(base + (size_t)so * D * es)[piece];
    }
    if (q < n_items_v) {
      const int dpl = q / (D * vq_row), rem = q % (D * vq_row);
      const int dd = rem / vq_row, piece = rem % vq_row;
      const int per = 16 / es;
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      for (int e = 0; e < per; ++e) {
        const int slot = piece * per + e;
        const int j = (dp_lo + dpl) * b + slot;
        const int sidx = src_of(j, s_ev, E);
        const int sp = sidx / b - dp_lo, so = sidx % b;
        const uint8_t* src = s_v + (size_t)sp * pb + ((size_t)dd * b + so) * es;
        if (es == 2) {
          const uint32_t x = *reinterpret_cast<const uint16_t*>(src);
          w[e >> 1] |= x << (16 * (e & 1));
        } else {
          w[e] = *reinterpret_cast<const uint32_t*>(src);
        }
      }
      vreg[it] = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
  __syncthreads();
  // write phase
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    const int q = threadIdx.x + it * CP_THREADS;
    if (q < n_items_k) {
      const int slot_g = q / kq_row, piece = q % kq_row;
      const int dp = dp_lo + slot_g / b, so = slot_g % b;
      reinterpret_cast<u32x4_t*>(P.k + pool_off(P, nbt[dp], h) + (size_t)so * D * es)[piece] = kreg[it];
    }
    if (q < n_items_v) {
      const int dpl = q / (D * vq_row), rem = q % (D * vq_row);
      const int dd = rem / vq_row, piece = rem % vq_row;
      reinterpret_cast<u32x4_t*>(P.v + pool_off(P, nbt[dp_lo + dpl], h) + (size_t)dd * b * es)[piece] = vreg[it];
    }
  }
}

int chunk_pages_for(int page_size, int D, int es) {
  const long pv = (long)page_size * D * es;
  int L = (int)(CP_LDS_BYTES / pv) - 1;
  return std::max(1, std::min(8, L));
}

}  // namespace

extern "C" size_t gp_compact_or_grow_workspace_size(int R, int H_kv, int max_pages, int page_size,
                                                   int C_max) {
  (void)C_max;
  if (R <= 0 || H_kv <= 0 || max_pages <= 0 || page_size <= 0) return 0;
  // sized for the widest supported element (fp32) and head_dim 128
  const int es = 4, D = 128;
  const int L = chunk_pages_for(page_size, D, es);
  const size_t max_chunks = (size_t)(max_pages + L - 1) / L;
  size_t bytes = 0;
  bytes += (size_t)R * sizeof(Info);
  bytes += (size_t)R * max_pages * 4 * 2;               // old_bt, rel
  bytes += (size_t)R * H_kv * MAX_EVICT * 4;
  bytes += (size_t)R * H_kv * 4;
  bytes = (bytes + 255) & ~(size_t)255;
  bytes += (size_t)R * H_kv * max_chunks * 2 * (size_t)page_size * D * es;
  return bytes;
}

extern "C" int gp_compact_or_grow(const int32_t* req_idx, int R, int B, const float* a_short,
                                  const float* a_long, int C_max, const int32_t* ws_counts,
                                  const int32_t* n_cand, double tau, int k_loc, int policy,
                                  const int32_t* policies, gp_kv_cache* kv, int32_t* block_tables,
                                  int32_t* n_pages, int max_pages, int32_t* context_lens,
                                  int32_t* refcount, int32_t* free_stack, int32_t* free_top,
                                  int32_t* decision, int32_t* kept_idx, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (R < 0 || B < 0 || C_max <= 0 || !kv || max_pages <= 0 || k_loc < 0) return GP_ERR_INVALID;
  if (R == 0) return GP_OK;
  if (!req_idx || !a_short || !a_long || !ws_counts || !n_cand || !block_tables || !n_pages ||
      !context_lens || !refcount || !free_stack || !free_top || !decision || !kept_idx || !kv->k ||
      !kv->v)
    return GP_ERR_INVALID;
  if (policy < GP_POLICY_AUTO || policy > GP_POLICY_INVERSE) return GP_ERR_INVALID;
  if (!(tau == tau)) return GP_ERR_INVALID;
  if (kv->page_tag) return GP_ERR_UNSUPPORTED;
  const int H_kv = kv->num_kv_heads, D = kv->head_dim, b = kv->page_size;
  if (H_kv <= 0 || kv->num_pages <= 0) return GP_ERR_INVALID;
  if (kv->dtype != GP_F32 && kv->dtype != GP_BF16) return GP_ERR_INVALID;
  if (D != 64 && D != 128) return GP_ERR_UNSUPPORTED;
  if (b != 16 && b != 32) return GP_ERR_UNSUPPORTED;
  if (C_max % 4 || C_max > SEL_THREADS * SEL_VPT) return GP_ERR_UNSUPPORTED;
  const size_t need = gp_compact_or_grow_workspace_size(R, H_kv, max_pages, b, C_max);
  if (!workspace || workspace_bytes < need) return GP_ERR_WORKSPACE;

  CParams P{};
  P.req_idx = req_idx;
  P.a_short = a_short;
  P.a_long = a_long;
  P.ws_counts = ws_counts;
  P.n_cand = n_cand;
  P.policies = policies;
  P.k = static_cast<uint8_t*>(kv->k);
  P.v = static_cast<uint8_t*>(kv->v);
  P.block_tables = block_tables;
  P.n_pages = n_pages;
  P.context_lens = context_lens;
  P.refcount = refcount;
  P.free_stack = free_stack;
  P.free_top = free_top;
  P.decision = decision;
  P.kept_idx = kept_idx;
  P.R = R;
  P.B = B;
  P.H_kv = H_kv;
  P.D = D;
  P.page_size = b;
  P.num_pages = kv->num_pages;
  P.max_pages = max_pages;
  P.C_max = C_max;
  P.k_loc = k_loc;
  P.policy = policy;
  P.es = kv->dtype == GP_F32 ? 4 : 2;
  P.tau = tau;
  P.chunk_pages = chunk_pages_for(b, D, P.es);
  P.max_chunks = (max_pages + P.chunk_pages - 1) / P.chunk_pages;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  size_t off = 0;
  P.info = reinterpret_cast<Info*>(ws + off);
  off += (size_t)R * sizeof(Info);
  P.old_bt = reinterpret_cast<int32_t*>(ws + off);
  off += (size_t)R * max_pages * 4;
  P.rel = reinterpret_cast<int32_t*>(ws + off);
  off += (size_t)R * max_pages * 4;
  P.ev = reinterpret_cast<int32_t*>(ws + off);
  off += (size_t)R * H_kv * MAX_EVICT * 4;
  P.dp0 = reinterpret_cast<int32_t*>(ws + off);
  off += (size_t)R * H_kv * 4;
  off = (off + 255) & ~(size_t)255;
  P.snap = ws + off;

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(decide_alloc_kernel, dim3(1), dim3(64), 0, s, P);
  GP_CHECK_LAUNCH();
  if (b == 16) hipLaunchKernelGGL(select_kernel<16>, dim3(H_kv, R), dim3(SEL_THREADS), 0, s, P);
  else hipLaunchKernelGGL(select_kernel<32>, dim3(H_kv, R), dim3(SEL_THREADS), 0, s, P);
  GP_CHECK_LAUNCH();
  hipLaunchKernelGGL(snapshot_kernel, dim3(P.max_chunks, H_kv, R), dim3(CP_THREADS), 0, s, P);
  GP_CHECK_LAUNCH();
  // items per thread: a chunk holds L pages of b key rows (D * es / 16 pieces each)
  const long items = ((long)P.chunk_pages * b * D * P.es / 16 + CP_THREADS - 1) / CP_THREADS;
  const size_t lds = (size_t)(P.chunk_pages + 1) * b * D * P.es;
  dim3 grid(P.max_chunks, H_kv, R);
  if (items <= 4) hipLaunchKernelGGL(compact_kernel<4>, grid, dim3(CP_THREADS), lds, s, P);
  else if (items <= 8) hipLaunchKernelGGL(compact_kernel<8>, grid, dim3(CP_THREADS), lds, s, P);
  else if (items <= 16) hipLaunchKernelGGL(compact_kernel<16>, grid, dim3(CP_THREADS), lds, s, P);
  else return GP_ERR_UNSUPPORTED;
  GP_CHECK_LAUNCH();
  return GP_OK;
}
