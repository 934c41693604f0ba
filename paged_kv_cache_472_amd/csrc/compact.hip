// Compress-or-grow at a page boundary for gfx950 (GrowPage Sec. 3.2 Eq. 8 decision, Sec. 3.3
// Eq. 9-10 selection and Compress & Hold / Grow by One Page, Sec. 4.2 and App. E.2 free-page pool,
// fallback and prefix-safe compaction, App. H.1 policies).
//
// Launches:
//   1. decide_alloc (one workgroup): requests in req_idx order. Decision from the exact comparison
//      of sum_h (K^S_h - K^L_h) / (H |C|) with tau; Grow pops the LIFO free stack; compression
//      pops one private page per shared page it must write (ascending logical order); released
//      references are applied after every pop of the call. Per-request work and the page checks
//      run in parallel; only the pop order is a serial scan.
//   2. select: s = max(a^S, a^L); the E evicted tokens (E <= page_size, 2 page_size for a
//      Shrink) are the E smallest of the unique keys (s, ~index) outside each page's k_loc
//      quota, which realises the (s desc, index asc) order exactly. Pages of 16 or 32 tokens:
//      three launches (chunk-local E smallest, their merge per request and KV head, kept_idx
//      written in parallel). Pages of 64..256 tokens: one workgroup per request and KV head,
//      radix selects for the page quotas and for the E-th smallest key.
//   3. chunk list + snapshot: the (request, head, chunk) items to rewrite are listed on the device;
//      compaction is a left shift by at most E slots, so a chunk of destination pages only reads
//      its own pages plus the first pages of the next chunk, which are saved first.
//   4. compact (resident workgroups striding over the list). Pages of 16 or 32 tokens, window by
//      window: tabulate the source slot of every destination slot, read all sources (key rows
//      into registers, value pages into LDS), barrier, write the window's destination pages.
//      Pages of 64..256 tokens: items also split the head dimension into 64-byte parts, and
//      each destination page is rewritten from an LDS ring of its source pages' value rows.
#include "common.h"

#include <atomic>
#include <climits>

namespace {

constexpr int MODE_NONE = 0;      // grow / no pages: kept_idx = -1 over |C|
constexpr int MODE_IDENTITY = 1;  // compress with nothing to evict: kept_idx = 0..|C|-1
constexpr int MODE_COMPACT = 2;
constexpr int SEL_T = 256;           // threads (candidate pages) per selection chunk
constexpr int MAX_CAND = 32768;      // largest candidate set
constexpr int SEL_MAX_CHUNKS = MAX_CAND / (SEL_T * 16);
constexpr int MAX_EVICT = 32;
constexpr int MAX_SPAN = 2;               // pages a compaction shifts by at most (Shrink: 2)
constexpr int SHRINK_MIN_CAPACITY = 1024; // tokens a Shrink must leave (GrowPage App. H.1)
constexpr int CHUNK_PAGES = 16;           // destination pages per compaction item (pages <= 32 tokens)
// calls whose 16-page items would number at most this many use 8-page items instead: the shift of
// a few requests then spreads over more workgroups (measured: one request of the long-reasoning
// 32/8-head batch 53 -> 47 us for its compress-or-grow; with 16 requests 16-page items are faster)
constexpr long SMALL_CALL_ITEMS = 512;
constexpr int WIDE_CHUNK_PAGES = 8;       // the same for larger pages: more, shorter items
constexpr int MAX_WINDOW_SLOTS = 8 * 32;  // LDS window pages (<= 8) x page size (<= 32)
constexpr int CP_THREADS = 256;
constexpr int CP_LDS_BYTES = 40 * 1024;  // source value pages of one window
constexpr int K_PIECES = 8;               // key pieces per thread and window
constexpr int V_PIECES = 12;              // staged value pieces per thread and window
constexpr int WIDE_MIN_PAGE = 64;         // page sizes from here on take the wide path
constexpr int WIDE_MAX_EVICT = 512;       // 2 pages of 256 tokens (Shrink)
constexpr int WIDE_T = 1024;              // threads of a wide selection workgroup
constexpr int WIDE_VPT = 32;              // candidates per thread (|C| <= 32768)
constexpr int WIDE_PART = 64;             // bytes of each key row one wide compaction item owns
constexpr int NUM_XCD = 8;                // accelerator dies of the chip, each with its own L2
constexpr int WIDE_MAX_PARTS = 128 * 4 / WIDE_PART;
constexpr int KEY_BITS = 46;              // 31 score bits above a 15-bit complemented index
// Candidate sets of at most this many selection chunks (SEL_T pages each) are selected by one
// workgroup per (request, KV head), chunk after chunk; longer ones by a workgroup per chunk and a
// merge (measured, 16 requests of up to 18K candidates: one workgroup per head 79 us, per chunk
// 36 us; one request of 2K candidates: 20 us against 26 us).
constexpr int FUSED_MAX_CHUNKS = 2;

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
  // mixed-precision cache (page_tag non-null): the fp8 and INT4 pools of the bf16 cache
  uint8_t* page_tag;
  uint8_t* k8;
  uint8_t* v8;
  float* k_scale;
  float* v_scale;
  uint8_t* k4;
  uint8_t* v4;
  uint16_t* k4_scale;
  uint16_t* v4_scale;
  int32_t* new_tag;   // [R, max_pages] tag of each rewritten destination page (mixed caches)
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
  int32_t* ev;        // [R, H_kv, max_evict]
  int32_t* dp0;       // [R, H_kv]
  unsigned long long* cand;  // [R, H_kv, SEL_MAX_CHUNKS, MAX_EVICT] chunk survivors
  int4* items;               // [R * H_kv * max_chunks * npart] (request * H_kv + head, chunk * npart + part,
                             //  request row r, the head's first changed page dp0)
  int32_t* n_items;          // [1]
  uint8_t* snap;      // [R, H_kv, max_chunks, MAX_SPAN, 2, page bytes]
  int R, B, H_kv, D, page_size, num_pages, max_pages, C_max, k_loc, policy, es;
  int L;              // layers whose working sets enter the decision (ws_counts [L, R, H_kv, 2])
  int span;           // pages a compaction of this call may shift by (1, or 2 when Shrink can occur)
  int chunk_pages, max_chunks, window_pages;
  int max_evict;      // evicted tokens per head the selection can hold (MAX_EVICT or 2 page_size)
  int npart;          // parts of the head dimension compacted apart (1 below WIDE_MIN_PAGE)
  int log_b, log_kq, log_vq, log_qpp;  // log2 of page size, 16-byte pieces per key row / value row / page
  int log_kpq;        // log2 of the 16-byte pieces of a key row one part owns
  int fuse_items;     // the selection appends the compaction items itself (one layer, uniform
  int split_check;    // the page checks of the requests ran in page_check_kernel (chk holds them)
  int32_t* chk;       // [R][2]: a page of the request is invalid or released; shared pages it writes
                      // cache); the allocator zeroes the item count before it
  double tau;
};

// A request's record and a work item, loaded by every lane of a workgroup alike and kept in
// scalar registers (the loops and branches they control are then scalar, not masked per lane).
__device__ __forceinline__ Info info_of(const CParams& P, int i) {
  const Info v = P.info[i];
  Info u;
  u.r = gp::uni(v.r);
  u.mode = gp::uni(v.mode);
  u.P = gp::uni(v.P);
  u.ctx_old = gp::uni(v.ctx_old);
  u.n = gp::uni(v.n);
  u.K_t = gp::uni(v.K_t);
  u.R_n = gp::uni(v.R_n);
  u.E = gp::uni(v.E);
  u.ctx_new = gp::uni(v.ctx_new);
  u.n_dest = gp::uni(v.n_dest);
  u.first_repl = gp::uni(v.first_repl);
  u.pad = 0;
  return u;
}
__device__ __forceinline__ int4 item_of(const CParams& P, int k) {
  const int4 v = P.items[k];
  return make_int4(gp::uni(v.x), gp::uni(v.y), gp::uni(v.z), gp::uni(v.w));
}

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

// Decision and page allocation for all boundary requests in one workgroup. The refcount of a
// page that sits in a block table does not change until the releases at the end of the call
// (pops only touch free pages), so everything except the order of the pops is computed for all
// requests at once; only a short register scan over the requests runs serially.
constexpr int DA_THREADS = 1024;
constexpr int DA_MAX_R = 1024;
constexpr int DA_PAIRS = 8;  // (request, page) pairs per allocator thread whose loads fly together
enum : int {
  F_VALID = 1, F_GROW = 2, F_SLOT = 4, F_EMPTY = 8, F_CHECK = 16, F_BAD = 32, F_SHRINK = 64
};
enum : int { O_NONE = 0, O_GROW = 1, O_IDENTITY = 2, O_COMPACT = 3 };

__device__ __forceinline__ int block_excl_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(x, o, GP_WAVE);
    if (lane >= o) x += t;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
  for (int k = 0; k < nw; ++k) {
    off += k < w ? s_w[k] : 0;
    tot += s_w[k];
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// Request i of the call: validity, primary decision (Eq. 8 over layers and KV heads) and
// compaction geometry. Its flags carry F_* bits and the eviction count E in bits 8 and up.
struct ReqPlan {
  Info inf;
  int flags, ndest, Pn, r;
};
__device__ ReqPlan plan_request(const CParams& P, int i) {
  const int b = P.page_size;
  Info inf = {};
  inf.mode = MODE_NONE;
  const int nc = P.n_cand[i];
  const int r = P.req_idx[i];
  // the working-set counts depend on the request's position only: their loads go out with
  // the first ones, eight (layer, head) pairs per step, every load before any use
  long long dsum = 0;  // sum over layers and KV heads of K^S - K^L
  bool bad_ws = false;
  const int nlh = P.L * P.H_kv;
  for (int base = 0; base < nlh; base += 8) {
    int ks[8], kl[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int lh = min(base + u, nlh - 1), l = lh / P.H_kv, h = lh - l * P.H_kv;
      const int32_t* w = P.ws_counts + (((size_t)l * P.R + i) * P.H_kv + h) * 2;
      ks[u] = w[0];
      kl[u] = w[1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // no branch, so the loads stay ahead of their uses
      const bool in = base + u < nlh;
      bad_ws |= in && (ks[u] < 0 || kl[u] < 0);
      dsum += in ? (long long)ks[u] - kl[u] : 0ll;
    }
  }
  inf.n = (nc > 0 && nc <= P.C_max) ? nc : 0;
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
  if (ok && n > 0 && bad_ws) ok = false;
  int flags = 0, ndest = 0;
  if (ok) {
    flags |= F_VALID;
    const int pol = P.policies ? P.policies[i] : P.policy;
    const long long HN = (long long)P.L * P.H_kv * n;  // Delta = dsum / HN
    bool want_grow, want_shrink = false;
    if (pol == GP_POLICY_FORCE_COMPRESS) want_grow = false;
    else if (pol == GP_POLICY_FORCE_GROW || n == 0) want_grow = true;
    else {
      const bool g = trend_exceeds(dsum, HN, P.tau);
      want_grow = (pol == GP_POLICY_INVERSE) ? !g : g;
      // GrowPage-Shrink (Eq. 13): Delta < -0.005 = -1/200, decided exactly
      if (!want_grow && pol == GP_POLICY_SHRINK) want_shrink = dsum * 200 < -HN;
    }
    // a Shrink must leave a capacity of at least SHRINK_MIN_CAPACITY tokens
    const bool shrink = want_shrink && Pn >= 2 && (long)(Pn - 1) * b >= SHRINK_MIN_CAPACITY;
    if (want_grow) flags |= F_GROW;
    if (shrink) flags |= F_SHRINK;
    if (Pn < P.max_pages) flags |= F_SLOT;
    if (n == 0) flags |= F_EMPTY;
    const int R_n = ctx - n;
    const int keep = shrink ? Pn - 2 : Pn - 1;  // pages of history plus recent tokens kept
    const int K_t = min(n, max(0, keep * b - R_n));
    const int E = n - K_t;
    inf.P = Pn;
    inf.ctx_old = ctx;
    inf.K_t = K_t;
    inf.R_n = R_n;
    inf.E = E;
    inf.ctx_new = K_t + R_n;
    ndest = (inf.ctx_new + b - 1) / b;
    inf.n_dest = ndest;
    if (E > 0 && E <= P.max_evict) flags |= F_CHECK;  // may compact: check its pages
    flags |= min(E, 65535) << 8;
  }
  ReqPlan out;
  out.inf = inf;
  out.flags = flags;
  out.ndest = ndest;
  out.Pn = Pn;
  out.r = r;
  return out;
}

// The page checks of phase B below for calls with many (request, page) pairs, one workgroup per
// request: the random refcount and tag loads of all pairs would otherwise queue on the one
// compute unit of the allocator. Writes the request's old block-table row, whether a page id is
// invalid or a page released, and how many pages it writes are shared.
constexpr int PC_THREADS = 256;
__global__ __launch_bounds__(PC_THREADS) void page_check_kernel(CParams P) {
  const int i = blockIdx.x, tid = threadIdx.x;
  __shared__ int s_pl[3];
  __shared__ int s_bad, s_cnt;
  if (tid == 0) {
    const ReqPlan pl = plan_request(P, i);
    s_pl[0] = (pl.flags & F_CHECK) ? pl.Pn : 0;
    s_pl[1] = pl.ndest;
    s_pl[2] = pl.r;
    s_bad = 0;
    s_cnt = 0;
  }
  __syncthreads();
  const int Pn = s_pl[0], ndest = s_pl[1], r = s_pl[2];
  int bad = 0, cnt = 0;
  for (int j0 = 0; j0 < Pn; j0 += 4 * PC_THREADS) {
    int pg[4], rc[4], tg[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = min(j0 + u * PC_THREADS + tid, Pn - 1);
      pg[u] = P.block_tables[(size_t)r * P.max_pages + j];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = (pg[u] >= 0 && pg[u] < P.num_pages) ? pg[u] : 0;
      rc[u] = P.refcount[pc];
      tg[u] = P.page_tag ? (int)P.page_tag[pc] : GP_TAG_BF16;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + u * PC_THREADS + tid;
      if (j >= Pn) continue;
      P.old_bt[(size_t)i * P.max_pages + j] = pg[u];
      if (pg[u] < 0 || pg[u] >= P.num_pages || tg[u] == GP_TAG_RELEASE) bad = 1;
      else if (j < ndest && rc[u] > 1) ++cnt;
    }
  }
  if (bad) atomicOr(&s_bad, 1);
  if (cnt) atomicAdd(&s_cnt, cnt);
  __syncthreads();
  if (tid == 0) {
    P.chk[2 * i] = s_bad;
    P.chk[2 * i + 1] = s_cnt;
  }
}

__global__ __launch_bounds__(DA_THREADS) void decide_alloc_kernel(CParams P) {
  const int tid = threadIdx.x;
  const int b = P.page_size, R = P.R;
  __shared__ int s_flags[DA_MAX_R], s_cnt[DA_MAX_R], s_pn[DA_MAX_R], s_ndest[DA_MAX_R];
  __shared__ unsigned char s_shr[DA_MAX_R];
  __shared__ int s_r[DA_MAX_R], s_top[DA_MAX_R], s_relbase[DA_MAX_R], s_pref[DA_MAX_R + 1];
  __shared__ int s_before[DA_MAX_R];  // shared pages of the compacting requests before request i
  __shared__ int s_first[DA_MAX_R];   // first replaced page of request i (INT_MAX: none)
  __shared__ int s_w[DA_THREADS / GP_WAVE];
  __shared__ int s_any_repl, s_top_end, s_nrel;

  // the stack top before the call, fetched while the requests are examined
  __shared__ int s_top0;
  if (tid == 0) {
    const int t0 = *P.free_top;
    s_top0 = (t0 < 0 || t0 > P.num_pages) ? 0 : t0;
    if (P.fuse_items) *P.n_items = 0;  // the selection appends the compaction items
  }

  // ---- A: per request (one thread each): validity, primary decision, compaction geometry
  for (int i = tid; i < R; i += DA_THREADS) {
    const ReqPlan pl = plan_request(P, i);
    const int flags = pl.flags, ndest = pl.ndest, Pn = pl.Pn, r = pl.r;
    const Info inf = pl.inf;
    if (i < DA_MAX_R) {
      s_flags[i] = flags;
      s_cnt[i] = 0;
      s_pn[i] = (flags & F_CHECK) ? Pn : 0;
      s_ndest[i] = ndest;
      s_r[i] = r;
    }
    P.info[i] = inf;
  }
  __syncthreads();

  // ---- B: every (request, page) pair of a request that may compact: all page ids valid,
  // count the shared ones among the pages it writes, keep a copy of the old block table row
  // (done by page_check_kernel for calls with many pairs)
  if (P.split_check) {
    for (int i = tid; i < R; i += DA_THREADS) {
      if (s_pn[i] > 0) {
        if (P.chk[2 * i]) s_flags[i] |= F_BAD;
        s_cnt[i] = P.chk[2 * i + 1];
      }
    }
  }
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < R; ++i) {
      s_pref[i] = acc;
      acc += s_pn[i];
    }
    s_pref[R] = acc;
  }
  __syncthreads();
  const int npairs = gp::uni(s_pref[R]);
  const int npairs_b = P.split_check ? 0 : npairs;  // pairs phase B checks here
  // (request, page) pair f: the last i with s_pref[i] <= f, and the page's index in the request
  auto pair_of = [&](int f, int* j) {
    int lo = 0, hi = R;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid] <= f) lo = mid; else hi = mid;
    }
    *j = f - s_pref[lo];
    return lo;
  };
  // DA_PAIRS pairs per thread at a time, every block-table load of the batch issued before the
  // dependent refcount and tag loads, and those before any use (past npairs: the last pair again,
  // unused; an invalid page id reads page 0, unused)
  for (int f0 = 0; f0 < npairs_b; f0 += DA_PAIRS * DA_THREADS) {
    int iv[DA_PAIRS], jv[DA_PAIRS], pgv[DA_PAIRS], rcv[DA_PAIRS], tgv[DA_PAIRS];
#pragma unroll
    for (int u = 0; u < DA_PAIRS; ++u) {
      iv[u] = pair_of(min(f0 + u * DA_THREADS + tid, npairs_b - 1), &jv[u]);
      pgv[u] = P.block_tables[(size_t)s_r[iv[u]] * P.max_pages + jv[u]];
    }
#pragma unroll
    for (int u = 0; u < DA_PAIRS; ++u) {
      const int pc = (pgv[u] >= 0 && pgv[u] < P.num_pages) ? pgv[u] : 0;
      rcv[u] = P.refcount[pc];
      tgv[u] = P.page_tag ? (int)P.page_tag[pc] : GP_TAG_BF16;
    }
#pragma unroll
    for (int u = 0; u < DA_PAIRS; ++u) {
      if (f0 + u * DA_THREADS + tid >= npairs_b) continue;
      const int i = iv[u], j = jv[u], pg = pgv[u];
      P.old_bt[(size_t)i * P.max_pages + j] = pg;
      if (pg < 0 || pg >= P.num_pages) atomicOr(&s_flags[i], F_BAD);
      // mixed caches: a request that must move tokens keeps its pages when one is released
      // (one tag per page cannot keep a released token masked among live ones)
      else if (tgv[u] == GP_TAG_RELEASE) atomicOr(&s_flags[i], F_BAD);
      else if (j < s_ndest[i] && rcv[u] > 1) atomicAdd(&s_cnt[i], 1);
    }
  }
  __syncthreads();

  // ---- C: allocation order (registers only): outcome, stack top before the pops, release base
  if (tid == 0) {
    int top = s_top0;
    int nrel = 0, any = 0, nsh = 0;
    for (int i = 0; i < R; ++i) {
      const int fl = s_flags[i];
      int out = O_NONE, dec = GP_DECISION_NO_PAGES;
      s_top[i] = top;
      s_relbase[i] = nrel;
      s_before[i] = nsh;
      s_first[i] = INT_MAX;
      bool shr = false;
      if (fl & F_VALID) {
        bool compress = true;
        int code = (fl & F_SHRINK) ? GP_DECISION_SHRINK : GP_DECISION_COMPRESS;
        if (fl & F_GROW) {
          if (top > 0 && (fl & F_SLOT)) {
            --top;
            out = O_GROW;
            dec = GP_DECISION_GROW;
            compress = false;
          } else if (fl & F_EMPTY) {
            compress = false;  // nothing to compress: NO_PAGES
          } else {
            code = GP_DECISION_GROW_FALLBACK_COMPRESS;
          }
        }
        if (compress) {
          const int E = fl >> 8;
          shr = (fl & F_SHRINK) != 0;
          if (E == 0) {
            out = O_IDENTITY;  // nothing moves; a Shrink still hands back its last page
            dec = code;
            nrel += shr ? 1 : 0;
          } else if (E > P.max_evict) {
            // unreachable for Compress & Hold (E <= page_size); a Shrink of 32-token pages
            dec = GP_DECISION_NO_PAGES;
            shr = false;
          } else if ((fl & F_BAD) || s_cnt[i] > top) {
            dec = GP_DECISION_NO_PAGES;
            shr = false;
          } else {
            out = O_COMPACT;
            dec = code;
            nsh += s_cnt[i];
            top -= s_cnt[i];
            nrel += s_cnt[i] + (shr ? 1 : 0);  // the Shrink's last page follows its replacements
            any |= s_cnt[i] > 0;
          }
        }
      }
      s_flags[i] = (out << 4) | dec;  // outcome for phase D
      s_shr[i] = shr ? 1 : 0;
    }
    s_top_end = top;
    s_nrel = nrel;
    s_any_repl = any;
  }
  __syncthreads();

  // ---- D: apply outcomes (one thread per request)
  for (int i = tid; i < R; i += DA_THREADS) {
    const int out = s_flags[i] >> 4, dec = s_flags[i] & 15;
    P.decision[i] = dec;
    const int r = s_r[i];
    if (out == O_GROW) {
      const int top = s_top[i];
      const int Pn = P.info[i].P;
      const int pg = P.free_stack[top - 1];
      P.free_stack[top - 1] = -1;
      P.block_tables[(size_t)r * P.max_pages + Pn] = pg;
      P.n_pages[r] = Pn + 1;
      if (pg >= 0 && pg < P.num_pages) P.refcount[pg] = 1;
      P.info[i].mode = MODE_NONE;
    } else if (out == O_IDENTITY) {
      P.info[i].mode = MODE_IDENTITY;
    } else if (out == O_COMPACT) {
      P.context_lens[r] = P.info[i].ctx_new;
      P.info[i].mode = MODE_COMPACT;
      P.info[i].first_repl = s_ndest[i];
    } else {
      P.info[i].mode = MODE_NONE;
    }
    if (s_shr[i]) {
      // Shrink: the last page leaves the block table (no destination page is that high) and is
      // released after this request's replaced pages
      const int Pn = P.info[i].P;
      const size_t e = (size_t)r * P.max_pages + Pn - 1;
      P.rel[s_relbase[i] + (out == O_COMPACT ? s_cnt[i] : 0)] = P.block_tables[e];
      P.block_tables[e] = -1;
      P.n_pages[r] = Pn - 1;
    }
  }
  // shared pages of compacting requests get private replacements, popped in ascending logical
  // order (an ordered scan over the pairs gives each its rank within its request)
  if (s_any_repl) {
    __syncthreads();
    int carry = 0;
    for (int f0 = 0; f0 < npairs; f0 += DA_PAIRS * DA_THREADS) {
      // thread tid takes the consecutive pairs f0 + DA_PAIRS tid + u, so one block scan of the
      // per-thread counts ranks the shared pairs in pair order; the loads of a batch fly together
      int iv[DA_PAIRS], jv[DA_PAIRS], pgv[DA_PAIRS];
      bool cv[DA_PAIRS], shv[DA_PAIRS];
#pragma unroll
      for (int u = 0; u < DA_PAIRS; ++u) {
        const int f = f0 + DA_PAIRS * tid + u;
        iv[u] = pair_of(min(f, npairs - 1), &jv[u]);
        cv[u] = f < npairs && (s_flags[iv[u]] >> 4) == O_COMPACT && jv[u] < s_ndest[iv[u]];
        pgv[u] = P.old_bt[(size_t)iv[u] * P.max_pages + jv[u]];
      }
      int nsh = 0;
#pragma unroll
      for (int u = 0; u < DA_PAIRS; ++u) {
        const int pc = (pgv[u] >= 0 && pgv[u] < P.num_pages) ? pgv[u] : 0;
        shv[u] = cv[u] && P.refcount[pc] > 1;
        nsh += shv[u] ? 1 : 0;
      }
      int total;
      int ex = carry + block_excl_scan(nsh, s_w, &total);
#pragma unroll
      for (int u = 0; u < DA_PAIRS; ++u) {
        if (!shv[u]) continue;
        const int i = iv[u], j = jv[u], pg = pgv[u];
        // shared pairs of earlier requests precede request i's in the scan
        const int rank = ex++ - s_before[i];
        const int top = s_top[i];
        const int np = P.free_stack[top - 1 - rank];
        P.free_stack[top - 1 - rank] = -1;
        P.rel[s_relbase[i] + rank] = pg;
        P.block_tables[(size_t)s_r[i] * P.max_pages + j] = np;
        if (np >= 0 && np < P.num_pages) P.refcount[np] = 1;
        atomicMin(&s_first[i], j);
      }
      carry += total;
    }
    __syncthreads();
    // a compacting request rewrites from its first replaced page at the latest
    for (int i = tid; i < R; i += DA_THREADS)
      if (s_first[i] != INT_MAX) P.info[i].first_repl = min(s_ndest[i], s_first[i]);
  }
  // the release list written above is read back below by other threads: with no release the
  // fence (a wait for every store of the kernel) is skipped
  if (s_nrel > 0) __threadfence();
  __syncthreads();

  // ---- E: release the replaced references after every pop, in release order, in chunks of
  // DA_THREADS: each release decrements its page; a page that reaches zero had all its remaining
  // references released by now, the last of them in this chunk, and is pushed at the position of
  // that last release among this chunk's zero-reaching releases
  __shared__ int s_rel[DA_THREADS], s_last[DA_THREADS];
  int top = s_top_end;
  const int nrel = s_nrel;
  for (int k0 = 0; k0 < nrel; k0 += DA_THREADS) {
    const int k = k0 + tid, cnt = min(DA_THREADS, nrel - k0);
    int pg = -1;
    if (tid < cnt) pg = P.rel[k];
    s_rel[tid] = pg;
    s_last[tid] = 0;
    __syncthreads();
    if (tid < cnt && pg >= 0 && pg < P.num_pages) {
      const int old = atomicSub(&P.refcount[pg], 1);
      if (old == 1) {
        int last = tid;
        for (int q = tid + 1; q < cnt; ++q)
          if (s_rel[q] == pg) last = q;
        s_last[last] = 1;
      }
    }
    __syncthreads();
    int total;
    const int pos = block_excl_scan(s_last[tid], s_w, &total);
    if (s_last[tid] && top + pos < P.num_pages) P.free_stack[top + pos] = s_rel[tid];
    top = min(P.num_pages, top + total);
    __syncthreads();
  }
  if (tid == 0) *P.free_top = top;
}

// minimum over the wave on the DPP path (lanes outside a broadcast's row mask see all-ones,
// the identity of the minimum)
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ unsigned long long dpp_min_step(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)v, CTRL, ROW_MASK, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xf, false);
  const unsigned long long t = ((unsigned long long)hi << 32) | lo;
  return t < v ? t : v;
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
  v = dpp_min_step<0xb1>(v);
  v = dpp_min_step<0x4e>(v);
  v = dpp_min_step<0x141>(v);
  v = dpp_min_step<0x140>(v);
  v = dpp_min_step<0x142, 0xa>(v);
  v = dpp_min_step<0x143, 0xc>(v);
  return gp::readlane63_u64(v);
}

// Larger and smaller of this lane's 64-bit key and lane (lane ^ J)'s (see gp::lane_pair_minmax:
// the two halves move alike, so a lane-swap pair holds the two keys whole)
template <int J>
__device__ __forceinline__ void lane_pair_minmax_u64(unsigned long long v, unsigned long long& hi,
                                                     unsigned long long& lo) {
  const uint32_t vl = (uint32_t)v, vh = (uint32_t)(v >> 32);
  unsigned long long a = v, b;
  if constexpr (J == 16 || J == 32) {
    const auto rl = J == 16 ? __builtin_amdgcn_permlane16_swap(vl, vl, false, false)
                            : __builtin_amdgcn_permlane32_swap(vl, vl, false, false);
    const auto rh = J == 16 ? __builtin_amdgcn_permlane16_swap(vh, vh, false, false)
                            : __builtin_amdgcn_permlane32_swap(vh, vh, false, false);
    a = ((unsigned long long)rh[0] << 32) | rl[0];
    b = ((unsigned long long)rh[1] << 32) | rl[1];
  } else {
    uint32_t bl, bh;
    if constexpr (J == 1) { bl = gp::dpp_u32<0xb1>(vl); bh = gp::dpp_u32<0xb1>(vh); }
    if constexpr (J == 2) { bl = gp::dpp_u32<0x4e>(vl); bh = gp::dpp_u32<0x4e>(vh); }
    if constexpr (J == 4) {
      bl = gp::dpp_u32<0x141>(gp::dpp_u32<0x1b>(vl));
      bh = gp::dpp_u32<0x141>(gp::dpp_u32<0x1b>(vh));
    }
    if constexpr (J == 8) {
      bl = gp::dpp_u32<0x140>(gp::dpp_u32<0x141>(vl));
      bh = gp::dpp_u32<0x140>(gp::dpp_u32<0x141>(vh));
    }
    b = ((unsigned long long)bh << 32) | bl;
  }
  hi = a > b ? a : b;
  lo = a > b ? b : a;
}

// One key per lane, sorted ascending over the 64 lanes (bitonic network).
template <int SIZE, int J>
__device__ __forceinline__ void sort64_step(unsigned long long& x, int lane) {
  unsigned long long hi, lo;
  lane_pair_minmax_u64<J>(x, hi, lo);
  const bool lower = (lane & J) == 0, asc = (lane & SIZE) == 0;
  x = lower == asc ? lo : hi;
  if constexpr (J > 1) sort64_step<SIZE, J / 2>(x, lane);
}
template <int SIZE = 64>
__device__ __forceinline__ unsigned long long sort64_asc(unsigned long long x, int lane) {
  if constexpr (SIZE > 2) x = sort64_asc<SIZE / 2>(x, lane);
  sort64_step<SIZE, SIZE / 2>(x, lane);
  return x;
}

// The E smallest of the K keys of every lane of a wave (E <= MAX_EVICT; all keys distinct;
// ~0 marks no key), ascending into out[0 .. E) (~0 past the wave's keys). The E-th smallest lane
// minimum bounds the E-th smallest key from above (E lanes hold a key at or below it), so when at
// most 64 keys lie at or below it they are listed in the wave's 64-key LDS scratch and sorted
// across the lanes; otherwise E rounds of wave minima.
template <int K>
__device__ __forceinline__ void wave_smallest(const unsigned long long (&key)[K], int E, int lane,
                                              unsigned long long* s_tmp, unsigned long long* out) {
  unsigned long long lm = ~0ull;
#pragma unroll
  for (int j = 0; j < K; ++j) lm = key[j] < lm ? key[j] : lm;
  const unsigned long long srt = sort64_asc(lm, lane);
  const unsigned long long T = gp::uni((uint64_t)(
      ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(srt >> 32), E - 1) << 32) |
      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)srt, E - 1)));
  uint32_t cnt = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) cnt += (key[j] <= T && key[j] != ~0ull) ? 1u : 0u;
  const uint32_t C = gp::uni(gp::wave_sum_u32(cnt));
  if (C <= GP_WAVE) {
    uint32_t base = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const bool c = key[j] <= T && key[j] != ~0ull;
      const uint64_t m = __builtin_amdgcn_ballot_w64(c);
      const uint32_t at = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (c) s_tmp[at] = key[j];
      base += (uint32_t)__builtin_popcountll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    unsigned long long v = (uint32_t)lane < C ? s_tmp[lane] : ~0ull;
    v = sort64_asc(v, lane);
    if (lane < E) out[lane] = v;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the scratch may be reused by this wave next
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    unsigned long long prev = 0;
    for (int e = 0; e < E; ++e) {
      unsigned long long m = ~0ull;
#pragma unroll
      for (int j = 0; j < K; ++j)
        if ((e == 0 || key[j] > prev) && key[j] < m) m = key[j];
      m = wave_min_u64(m);
      prev = m;
      if (lane == 0) out[e] = m;
    }
  }
}

// Compaction items of one compacting head, appended to the work list: the chunks from the one
// holding its first changed page dp0 to the one holding its last destination page, each with every
// part of the head dimension. The order of the list does not matter (items never share bytes, and
// the pages a chunk reads from the next one are saved before any item runs).
__device__ __forceinline__ void append_items(const CParams& P, int i, int h, int r, int dp0, int n_dest) {
  const int L = P.chunk_pages;
  if (dp0 >= n_dest) return;
  const int c0 = dp0 / L * P.npart;
  const int cnt = ((n_dest + L - 1) / L - dp0 / L) * P.npart;
  const int off = atomicAdd(P.n_items, cnt);
  for (int k = 0; k < cnt; ++k) P.items[off + k] = make_int4(i * P.H_kv + h, c0 + k, r, dp0);
}

// kept_idx over the output positions [p0, p1), written by consecutive threads: position p holds
// the p-th kept candidate, p + #{k : ev[k] - k <= p} (ev the E evicted candidates, ascending, so
// ev[k] - k never decreases); the thresholds ev[k] - k are wave-uniform
__device__ __forceinline__ void write_kept(int32_t* out, int p0, int p1, const int* s_ev, int E,
                                           int tid, int nthreads) {
  int thr[MAX_EVICT];
#pragma unroll
  for (int k = 0; k < MAX_EVICT; ++k) thr[k] = gp::uni(k < E ? s_ev[k] - k : INT_MAX);
  for (int p = p0 + tid; p < p1; p += nthreads) {
    int c = 0;
#pragma unroll
    for (int k0 = 0; k0 < MAX_EVICT; k0 += 8) {
      if (k0 < E) {
#pragma unroll
        for (int k = k0; k < k0 + 8; ++k) c += thr[k] <= p ? 1 : 0;
      }
    }
    out[p] = p + c;
  }
}

// Selection (Eq. 9-10) in two short launches over chunks of SEL_T pages (one page per
// thread, so the k_loc quota of a page is ranked in registers).
//   select_local: per chunk, the E smallest eviction keys (s, ~index) of the chunk: each wave
//                 finds its own E smallest with shuffles, then one wave picks the E smallest of
//                 the 4 * E survivors.
//   select_write: per chunk, first the E smallest of all of its head's chunk survivors (the
//                 evicted tokens, sorted by token index; chunk 0 also records them and the first
//                 destination page that changes), then kept_idx: kept token t goes to position
//                 t - #(evicted < t).
// Keys are unique, so the result is exactly the (s desc, index asc) order whatever the split.
template <int PB>
__global__ __launch_bounds__(SEL_T) void select_local_kernel(CParams P) {
  constexpr int b = PB;
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Info inf = info_of(P, i);
  const int n = inf.n;
  if (inf.mode != MODE_COMPACT || c * SEL_T * b >= n) return;
  const int K_t = inf.K_t, E = inf.E;
  const int t0 = (c * SEL_T + threadIdx.x) * b;  // first candidate of this thread's page
  const float* as = P.a_short + ((size_t)i * P.H_kv + h) * P.C_max;
  const float* al = P.a_long + ((size_t)i * P.H_kv + h) * P.C_max;
  uint32_t sv[b];
#pragma unroll
  for (int j = 0; j < b; j += 4) {
    if (t0 < n) {  // pages are whole: t0 < n covers all b candidates
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(as + t0 + j);
      const f32x4_t y = *reinterpret_cast<const f32x4_t*>(al + t0 + j);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sv[j + e] = max(__float_as_uint(x[e]) & 0x7fffffffu, __float_as_uint(y[e]) & 0x7fffffffu);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) sv[j + e] = 0u;
    }
  }
  const int kloc = min(P.k_loc, b);
  const long n_loc = (long)(n / b) * kloc;
  const bool pool_all = n_loc >= K_t;  // |S_loc| >= K_t: S is the K_t best of all of C
  unsigned long long key[b];
#pragma unroll
  for (int j = 0; j < b; ++j) {
    bool cand = t0 < n;
    if (cand && !pool_all) {
      // rank of candidate j inside its page under (s desc, index asc): the k_loc best stay
      int rank = 0;
#pragma unroll
      for (int u = 0; u < b; ++u) rank += (sv[u] > sv[j] || (sv[u] == sv[j] && u < j)) ? 1 : 0;
      cand = rank >= kloc;
    }
    key[j] = cand ? (((unsigned long long)sv[j] << 32) | (0xffffffffu - (uint32_t)(t0 + j))) : ~0ull;
  }
  constexpr int NW = SEL_T / GP_WAVE;
  __shared__ unsigned long long s_cand[NW * MAX_EVICT];
  __shared__ unsigned long long s_tmp[NW * GP_WAVE];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  wave_smallest<b>(key, E, lane, s_tmp + wv * GP_WAVE, s_cand + wv * MAX_EVICT);
  __syncthreads();
  if (wv == 0) {
    constexpr int PER = NW * MAX_EVICT / GP_WAVE;
    unsigned long long cv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = lane + GP_WAVE * k;
      cv[k] = (idx % MAX_EVICT) < E ? s_cand[idx] : ~0ull;
    }
    unsigned long long* dst = P.cand + (((size_t)i * P.H_kv + h) * SEL_MAX_CHUNKS + c) * MAX_EVICT;
    wave_smallest<PER>(cv, E, lane, s_tmp, dst);
  }
}

// The E smallest eviction keys of a head over the survivors of its chunks (one wave), as the
// evicted tokens sorted by index into s_ev[0 .. E) (INT_MAX past E)
__device__ __forceinline__ void merge_evicted(const CParams& P, int i, int h, int n, int E, int lane,
                                              unsigned long long* s_tmp, unsigned long long* s_best,
                                              int* s_ev) {
  const int b = P.page_size;
  const int nch = (n + SEL_T * b - 1) / (SEL_T * b);
  const unsigned long long* src = P.cand + ((size_t)i * P.H_kv + h) * SEL_MAX_CHUNKS * MAX_EVICT;
  constexpr int PER = SEL_MAX_CHUNKS * MAX_EVICT / GP_WAVE;
  unsigned long long cv[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = lane + GP_WAVE * k;  // chunk idx / MAX_EVICT, rank idx % MAX_EVICT
    cv[k] = (idx / MAX_EVICT < nch && (idx % MAX_EVICT) < E) ? src[idx] : ~0ull;
  }
  wave_smallest<PER>(cv, E, lane, s_tmp, s_best);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // lane e < E: the e-th evicted token (by key); its rank by index places it
  const int tok = lane < E ? (int)(0xffffffffu - (uint32_t)(s_best[lane] & 0xffffffffu)) : INT_MAX;
  int rank = 0;
  for (int e = 0; e < E; ++e) {
    const int o = __shfl(tok, e, GP_WAVE);
    rank += o < tok ? 1 : 0;
  }
  if (lane < E) s_ev[rank] = tok;
  else if (lane < MAX_EVICT) s_ev[lane] = INT_MAX;
}

template <int PB>
__global__ __launch_bounds__(SEL_T) void select_write_kernel(CParams P) {
  constexpr int b = PB;
  const int c = blockIdx.x, h = blockIdx.y, i = blockIdx.z;
  const Info inf = info_of(P, i);
  const int n = inf.n;
  if (c * SEL_T * b >= n) return;
  int32_t* out = P.kept_idx + ((size_t)i * P.H_kv + h) * P.C_max;
  const int t0 = (c * SEL_T + threadIdx.x) * b;
  if (inf.mode != MODE_COMPACT) {
    if (t0 < n)
      for (int j = 0; j < b; ++j) out[t0 + j] = inf.mode == MODE_IDENTITY ? t0 + j : -1;
    return;
  }
  const int E = inf.E;
  // every chunk's workgroup merges the head's chunk survivors itself (a few hundred keys in one
  // wave), which saves a launch between the local selection and this one; chunk 0's writes the
  // evicted list, the first changed page and the compaction items
  __shared__ int s_ev[MAX_EVICT];
  __shared__ unsigned long long s_tmp[GP_WAVE], s_best[MAX_EVICT];
  if (threadIdx.x < GP_WAVE) merge_evicted(P, i, h, n, E, threadIdx.x, s_tmp, s_best, s_ev);
  __syncthreads();
  if (c == 0) {
    if (threadIdx.x < E) {
      P.ev[((size_t)i * P.H_kv + h) * P.max_evict + threadIdx.x] = s_ev[threadIdx.x];
      out[inf.K_t + threadIdx.x] = -1;
    }
    if (threadIdx.x == 0) {
      const int dp0 = min(s_ev[0] / b, inf.first_repl);
      P.dp0[(size_t)i * P.H_kv + h] = dp0;
      if (P.fuse_items) append_items(P, i, h, inf.r, dp0, inf.n_dest);
    }
  }
  // this chunk's kept candidates: the output positions between those of its first candidate and
  // of the next chunk's
  const int ta = c * SEL_T * b, tb = min(n, ta + SEL_T * b);
  int ea = 0, eb = 0;
#pragma unroll
  for (int e = 0; e < MAX_EVICT; ++e) {
    ea += s_ev[e] < ta ? 1 : 0;
    eb += s_ev[e] < tb ? 1 : 0;
  }
  write_kept(out, ta - ea, tb - eb, s_ev, E, threadIdx.x, SEL_T);
}

// The three selection steps in one workgroup per (request, KV head), for calls with few requests:
// the chunks of SEL_T pages are taken one after another, each leaving its E smallest eviction keys
// merged into a running set of E in LDS; then the evicted list, the first changed page, kept_idx
// and (with fuse_items) the compaction items of the head.
template <int PB>
__global__ __launch_bounds__(SEL_T) void select_fused_kernel(CParams P) {
  constexpr int b = PB;
  constexpr int NW = SEL_T / GP_WAVE;
  const int h = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const float* as = P.a_short + ((size_t)i * P.H_kv + h) * P.C_max;
  const float* al = P.a_long + ((size_t)i * P.H_kv + h) * P.C_max;
  // the first chunk's scores go out with the request's plan (their addresses do not depend on
  // it; indexes are kept inside the row and pages past |C| are dropped below)
  f32x4_t x0[b / 4], y0[b / 4];
#pragma unroll
  for (int j = 0; j < b; j += 4) {
    const int t = min(tid * b + j, P.C_max - 4);
    x0[j / 4] = *reinterpret_cast<const f32x4_t*>(as + t);
    y0[j / 4] = *reinterpret_cast<const f32x4_t*>(al + t);
  }
  const Info inf = info_of(P, i);
  const int n = inf.n;
  int32_t* out = P.kept_idx + ((size_t)i * P.H_kv + h) * P.C_max;
  if (inf.mode != MODE_COMPACT) {
    for (int t = tid; t < n; t += SEL_T) out[t] = inf.mode == MODE_IDENTITY ? t : -1;
    return;
  }
  const int K_t = inf.K_t, E = inf.E;
  const int kloc = min(P.k_loc, b);
  const bool pool_all = (long)(n / b) * kloc >= K_t;  // |S_loc| >= K_t: the K_t best of all of C
  const int nch = (n + SEL_T * b - 1) / (SEL_T * b);
  __shared__ unsigned long long s_cand[NW * MAX_EVICT];
  __shared__ unsigned long long s_best[MAX_EVICT];
  __shared__ unsigned long long s_tmp[NW * GP_WAVE];
  __shared__ int s_ev[MAX_EVICT];
  for (int c = 0; c < nch; ++c) {
    const int t0 = (c * SEL_T + tid) * b;  // first candidate of this thread's page
    uint32_t sv[b];
#pragma unroll
    for (int j = 0; j < b; j += 4) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
      if (t0 < n) {  // pages are whole: t0 < n covers all b candidates
        if (c == 0) {
          x = x0[j / 4];
          y = y0[j / 4];
        } else {
          x = *reinterpret_cast<const f32x4_t*>(as + t0 + j);
          y = *reinterpret_cast<const f32x4_t*>(al + t0 + j);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sv[j + e] = max(__float_as_uint(x[e]) & 0x7fffffffu, __float_as_uint(y[e]) & 0x7fffffffu);
    }
    unsigned long long key[b];
#pragma unroll
    for (int j = 0; j < b; ++j) {
      bool cand = t0 < n;
      if (cand && !pool_all) {
        // rank of candidate j inside its page under (s desc, index asc): the k_loc best stay
        int rank = 0;
#pragma unroll
        for (int u = 0; u < b; ++u) rank += (sv[u] > sv[j] || (sv[u] == sv[j] && u < j)) ? 1 : 0;
        cand = rank >= kloc;
      }
      key[j] = cand ? (((unsigned long long)sv[j] << 32) | (0xffffffffu - (uint32_t)(t0 + j))) : ~0ull;
    }
    // each wave's E smallest
    wave_smallest<b>(key, E, lane, s_tmp + wv * GP_WAVE, s_cand + wv * MAX_EVICT);
    __syncthreads();
    if (wv == 0) {
      // the E smallest of the waves' survivors and the running set
      constexpr int TOT = (NW + 1) * MAX_EVICT;
      constexpr int PER = (TOT + GP_WAVE - 1) / GP_WAVE;
      unsigned long long cv[PER];
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int idx = lane + GP_WAVE * k;
        unsigned long long v = ~0ull;
        if (idx < NW * MAX_EVICT) v = (idx % MAX_EVICT) < E ? s_cand[idx] : ~0ull;
        else if (idx < TOT && c > 0 && idx - NW * MAX_EVICT < E) v = s_best[idx - NW * MAX_EVICT];
        cv[k] = v;
      }
      wave_smallest<PER>(cv, E, lane, s_tmp, s_best);
    }
    __syncthreads();
  }
  // the evicted tokens sorted by index: lane e ranks the e-th smallest key's token among the E
  if (wv == 0) {
    const int tok = lane < E ? (int)(0xffffffffu - (uint32_t)(s_best[lane] & 0xffffffffu)) : INT_MAX;
    int rank = 0;
    for (int e = 0; e < E; ++e) rank += __shfl(tok, e, GP_WAVE) < tok ? 1 : 0;
    if (lane < E) s_ev[rank] = tok;
  }
  __syncthreads();
  if (tid < E) P.ev[((size_t)i * P.H_kv + h) * P.max_evict + tid] = s_ev[tid];
  if (tid < E) out[K_t + tid] = -1;
  const int dp0 = min(s_ev[0] / b, inf.first_repl);
  if (tid == 0) {
    P.dp0[(size_t)i * P.H_kv + h] = dp0;
    if (P.fuse_items) append_items(P, i, h, inf.r, dp0, inf.n_dest);
  }
  // kept_idx: the K_t kept candidates in order
  write_kept(out, 0, K_t, s_ev, E, tid, SEL_T);
}

// Selection for pages of 64..256 tokens (up to 2 page_size evictions): one workgroup per
// (request, KV head), WIDE_VPT consecutive candidates per thread. A key holds the score bits
// above the complemented token index, so a larger key is a better token under (s desc,
// index asc) and all keys differ. The k_loc quota of a page is every key at or above the
// page's k_loc-th largest, found by a bitwise radix select over the LPP lanes that hold the
// page; the evicted tokens are the keys outside the quotas up to the E-th smallest of them,
// found by a bitwise radix select over the workgroup. Writes the ascending evicted list, the
// first changed destination page and kept_idx.
template <int LPP>  // lanes per page: page_size / WIDE_VPT
__global__ __launch_bounds__(WIDE_T) void select_wide_kernel(CParams P) {
  const int h = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const Info inf = info_of(P, i);
  const int n = inf.n;
  int32_t* out = P.kept_idx + ((size_t)i * P.H_kv + h) * P.C_max;
  if (inf.mode != MODE_COMPACT) {
    for (int t = tid; t < n; t += WIDE_T) out[t] = inf.mode == MODE_IDENTITY ? t : -1;
    return;
  }
  const int K_t = inf.K_t, E = inf.E, b = P.page_size;
  const int t0 = tid * WIDE_VPT;
  const bool live = t0 < n;  // |C| is a multiple of the page size, so of WIDE_VPT
  const float* as = P.a_short + ((size_t)i * P.H_kv + h) * P.C_max;
  const float* al = P.a_long + ((size_t)i * P.H_kv + h) * P.C_max;
  unsigned long long key[WIDE_VPT];
#pragma unroll
  for (int j = 0; j < WIDE_VPT; j += 4) {
    f32x4_t x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      x = *reinterpret_cast<const f32x4_t*>(as + t0 + j);
      y = *reinterpret_cast<const f32x4_t*>(al + t0 + j);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sv = max(__float_as_uint(x[e]) & 0x7fffffffu, __float_as_uint(y[e]) & 0x7fffffffu);
      key[j + e] = ((unsigned long long)sv << 15) | (uint32_t)(0x7fff - ((t0 + j + e) & 0x7fff));
    }
  }
  const int kloc = min(P.k_loc, b);
  const long n_loc = (long)(n / b) * kloc;
  if (n_loc < K_t && kloc > 0 && live) {
    // the page's kloc-th largest key: the largest x with #{keys >= x} >= kloc (the lanes of a
    // page are live together, and waves past |C| skip the search)
    unsigned long long x = 0;
    for (int bit = KEY_BITS - 1; bit >= 0; --bit) {
      const unsigned long long c = x | (1ull << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < WIDE_VPT; ++j) cnt += key[j] >= c ? 1 : 0;
#pragma unroll
      for (int o = 1; o < LPP; o <<= 1) cnt += __shfl_xor(cnt, o, GP_WAVE);
      if (cnt >= kloc) x = c;
    }
#pragma unroll
    for (int j = 0; j < WIDE_VPT; ++j)
      if (key[j] >= x) key[j] = ~0ull;  // in the quota: never evicted
  }
  // otherwise |S_loc| >= K_t and S is the K_t best of all of C: every candidate may go
  if (!live) {
#pragma unroll
    for (int j = 0; j < WIDE_VPT; ++j) key[j] = ~0ull;
  }
  // the E-th smallest remaining key: the largest x with #{keys < x} < E
  constexpr int NW = WIDE_T / GP_WAVE;
  __shared__ int s_part[2][NW];
  __shared__ int s_w[NW];
  const int lane = tid & 63, wv = tid >> 6;
  unsigned long long x = 0;
  for (int bit = KEY_BITS - 1, it = 0; bit >= 0; --bit, ++it) {
    const unsigned long long c = x | (1ull << bit);
    int cnt = 0;
    if (live) {  // waves past |C| only take part in the reduction
#pragma unroll
      for (int j = 0; j < WIDE_VPT; ++j) cnt += key[j] < c ? 1 : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, GP_WAVE);
    if (lane == 0) s_part[it & 1][wv] = cnt;
    __syncthreads();  // one barrier per step: the two buffers alternate
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_part[it & 1][w];
    if (tot < E) x = c;
  }
  uint32_t evm = 0;  // bit j: candidate t0 + j is evicted
#pragma unroll
  for (int j = 0; j < WIDE_VPT; ++j) evm |= (key[j] <= x ? 1u : 0u) << j;
  int total;
  const int ex = block_excl_scan(__popc(evm), s_w, &total);  // total == E
  int32_t* ev = P.ev + ((size_t)i * P.H_kv + h) * P.max_evict;
  if (evm) {
    int k = ex;
    for (int j = 0; j < WIDE_VPT; ++j)
      if ((evm >> j) & 1u) ev[k++] = t0 + j;
    if (ex == 0) {
      const int dp0 = min((t0 + __ffs(evm) - 1) / b, inf.first_repl);
      P.dp0[(size_t)i * P.H_kv + h] = dp0;
      if (P.fuse_items) append_items(P, i, h, inf.r, dp0, inf.n_dest);
    }
  }
  if (live) {
    int before = ex;  // evicted tokens below t0 + j
    for (int j = 0; j < WIDE_VPT; ++j) {
      if ((evm >> j) & 1u) ++before;
      else out[t0 + j - before] = t0 + j;
    }
  }
  if (tid < E) out[K_t + tid] = -1;
}

// page bytes of one KV head: keys [b][D], values [D][b]
__device__ __forceinline__ size_t page_bytes(const CParams& P) { return (size_t)P.page_size * P.D * P.es; }
__device__ __forceinline__ size_t pool_off(const CParams& P, int pg, int h) {
  return ((size_t)pg * P.H_kv + h) * page_bytes(P);
}
// saved page lp of a head: chunk lp / chunk_pages, slot lp % chunk_pages (< MAX_SPAN)
__device__ __forceinline__ uint8_t* snap_ptr(const CParams& P, int i, int h, int lp, int which) {
  const int c = lp / P.chunk_pages, s = lp % P.chunk_pages;
  return P.snap + (((((size_t)i * P.H_kv + h) * P.max_chunks + c) * MAX_SPAN + s) * 2 + which) *
                      page_bytes(P);
}
// does chunk c read logical page lp from the snapshot? Only the first pages of the next chunk
// that its sources reach, and only those that chunk rewrites (pages below n_dest): the workgroup
// of chunk c + 1 may have rewritten them by the time chunk c reads them. Pages of chunk c itself
// are read before the same workgroup writes them. A request evicting E tokens shifts a slot by at
// most E, so its sources reach ceil(E / b) pages past a destination page (one for a Compress, two
// for a Shrink; the call's span is the most any request may need): a page past those is never
// used, whatever it holds when read.
__device__ __forceinline__ bool from_snapshot(const CParams& P, int lp, int c, const Info& inf) {
  const int first = (c + 1) * P.chunk_pages;
  const int reach = min(P.span, (inf.E + (1 << P.log_b) - 1) >> P.log_b);
  return lp >= first && lp < first + reach && lp < inf.n_dest;
}

// List of the (request, head, chunk, part) items that compaction rewrites: for a compacting head
// the chunks from the one holding its first changed page to the one holding its last destination
// page, each with every part of the head dimension (one part below WIDE_MIN_PAGE).
__global__ __launch_bounds__(DA_THREADS) void chunk_list_kernel(CParams P) {
  __shared__ int s_w[DA_THREADS / GP_WAVE];
  const int L = P.chunk_pages, n = P.R * P.H_kv;
  int carry = 0;
  for (int base = 0; base < n; base += DA_THREADS) {
    const int ih = base + threadIdx.x;
    int c0 = 0, cnt = 0, r = 0, dp0 = 0;
    if (ih < n) {
      const Info inf = P.info[ih / P.H_kv];
      if (inf.mode == MODE_COMPACT) {
        r = inf.r;
        dp0 = P.dp0[ih];
        if (dp0 < inf.n_dest) {
          c0 = dp0 / L * P.npart;
          cnt = ((inf.n_dest + L - 1) / L - dp0 / L) * P.npart;
        }
      }
    }
    int total;
    const int off = carry + block_excl_scan(cnt, s_w, &total);
    for (int k = 0; k < cnt; ++k) P.items[off + k] = make_int4(ih, c0 + k, r, dp0);  // chunk * npart + part
    carry += total;
  }
  if (threadIdx.x == 0) *P.n_items = carry;
}

// The first `span` pages of the next chunk, saved before any chunk is rewritten (they are that
// chunk's to rewrite, and this chunk's last source pages): the bytes of the item's part, i.e.
// its slice of every key row and its value rows. Workgroups stride over the work list.
__global__ __launch_bounds__(CP_THREADS) void snapshot_kernel(CParams P) {
  const int n_items = gp::uni(*P.n_items);
  const int krow = P.D * P.es, kb = krow / P.npart;   // key row bytes, of them the part's
  const size_t vb = page_bytes(P) / P.npart;           // value bytes of the part (contiguous rows)
  const int lkpq = P.log_kpq, nkq = P.page_size << lkpq;
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int4 item = item_of(P, it);
    const int i = item.x / P.H_kv, h = item.x % P.H_kv;
    const int c = item.y / P.npart, part = item.y % P.npart;
    // the old block-table entries of the next chunk's first pages load with the request's record
    // (indexes kept inside the row; pages the snapshot skips are dropped)
    int pgs[MAX_SPAN];
#pragma unroll
    for (int s = 0; s < MAX_SPAN; ++s)
      pgs[s] = P.old_bt[(size_t)i * P.max_pages + min((c + 1) * P.chunk_pages + s, P.max_pages - 1)];
    const Info inf = info_of(P, i);
    for (int s = 0; s < P.span; ++s) {
      const int lp = (c + 1) * P.chunk_pages + s;
      if (!from_snapshot(P, lp, c, inf)) continue;  // uniform over the workgroup
      const int pg = gp::uni(s == 0 ? pgs[0] : pgs[MAX_SPAN - 1]);
      const uint8_t* ks = P.k + pool_off(P, pg, h) + (size_t)part * kb;
      const uint8_t* vs = P.v + pool_off(P, pg, h) + (size_t)part * vb;
      uint8_t* kd = snap_ptr(P, i, h, lp, 0) + (size_t)part * kb;
      uint8_t* vd = snap_ptr(P, i, h, lp, 1) + (size_t)part * vb;
      // four key and four value pieces per thread in flight before any is stored
      auto key_at = [&](int q) {
        return (size_t)(q >> lkpq) * krow + (size_t)(q & ((1 << lkpq) - 1)) * 16;
      };
      const int nvq = (int)(vb / 16);
      for (int q0 = threadIdx.x; q0 < max(nkq, nvq); q0 += 4 * CP_THREADS) {
        u32x4_t xk[4], xv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          xk[u] = *reinterpret_cast<const u32x4_t*>(ks + key_at(min(q0 + u * CP_THREADS, nkq - 1)));
          xv[u] = reinterpret_cast<const u32x4_t*>(vs)[min(q0 + u * CP_THREADS, nvq - 1)];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (q0 + u * CP_THREADS < nkq) *reinterpret_cast<u32x4_t*>(kd + key_at(q0 + u * CP_THREADS)) = xk[u];
          if (q0 + u * CP_THREADS < nvq) reinterpret_cast<u32x4_t*>(vd)[q0 + u * CP_THREADS] = xv[u];
        }
      }
    }
  }
}

// Barrier for LDS hand-offs only: waits for this wave's LDS operations, not for its global
// stores, so a window's writes drain while the next window's reads are in flight. Windows and
// items of a workgroup never read bytes that another of its windows writes (see compact_kernel),
// so the global stores need no ordering inside the kernel.
constexpr long long NO_SRC = LLONG_MIN;  // no source page (past the request's old pages)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
}

// Destination slot j of a compacted head takes source slot j + #{k : ev[k] - k <= j} (ev the
// ascending evicted candidates): the j-th kept candidate, then the recent tokens. A workgroup
// owns a chunk of destination pages and walks it left to right in windows. Per window it
// tabulates the source slot of every destination slot, reads the key rows it will write into
// registers (rows are contiguous, 16 bytes per lane), stages the source value pages (token-
// contiguous inside a page, so a gather needs them whole) in LDS, and only then writes the
// window's destination pages. A shift of at most `span` pages means a window of destination
// pages [w0, w1) reads source pages [w0, w1 + span - 1]; inside a chunk those are not yet
// rewritten when read, and the first `span` pages of the next chunk, which another workgroup
// rewrites, come from the snapshot.
__global__ __launch_bounds__(CP_THREADS) void compact_kernel(CParams P) {
  const int n_items = gp::uni(*P.n_items);
  for (int item_k = blockIdx.x; item_k < n_items; item_k += gridDim.x) {
  lds_barrier();  // the previous item is done with the tables and LDS
  const int4 item = item_of(P, item_k);
  const int i = item.x / P.H_kv, h = item.x % P.H_kv, c = item.y, r = item.z;
  const int L = P.chunk_pages, W = P.window_pages, D = P.D, es = P.es;
  const int lb = P.log_b, b = 1 << lb;
  const int dp_lo = max(item.w, c * L);
  // the item's own loads go out together (the item carries the request row and dp0): the
  // request's record, the head's evicted list and the old and new block-table entries of pages
  // dp_lo .. (indexes kept inside the rows; what lies past the chunk or the old pages is
  // dropped once the record is in)
  const Info inf = info_of(P, i);
  const int t = threadIdx.x;
  const int ev_t = P.ev[((size_t)i * P.H_kv + h) * P.max_evict + min(t, P.max_evict - 1)];
  const int lpc = min(dp_lo + t, P.max_pages - 1);
  const int old_pg = P.old_bt[(size_t)i * P.max_pages + lpc];
  const int new_pg = P.block_tables[(size_t)r * P.max_pages + lpc];
  const int dp_hi = min((c + 1) * L, inf.n_dest);
  __shared__ int s_thr[MAX_EVICT];
  __shared__ int s_src[MAX_WINDOW_SLOTS];
  // source pages dp_lo .. dp_hi + span - 1: byte offset of the (page, head) key block from the
  // key pool's base and of the value block from the value pool's base, in the pool or in the
  // snapshot (NO_SRC past the old pages); destination pages dp_lo .. dp_hi - 1: pool byte offset.
  // Offsets from the pool pointers keep every access in the global address space.
  __shared__ long long s_ksrc[CHUNK_PAGES + MAX_SPAN];
  __shared__ long long s_vsrc[CHUNK_PAGES + MAX_SPAN];
  __shared__ long long s_doff[CHUNK_PAGES];
  extern __shared__ __align__(16) uint8_t s_v[];  // value pages of the window
  const int E = inf.E;
  const size_t pb = page_bytes(P);
  if (t < MAX_EVICT) s_thr[t] = t < E ? ev_t - t : INT_MAX;
  if (t < dp_hi - dp_lo + P.span) {
    const int lp = dp_lo + t;
    long long ks = NO_SRC, vs = NO_SRC;
    if (lp < inf.P) {
      if (from_snapshot(P, lp, c, inf)) {
        ks = (long long)((intptr_t)snap_ptr(P, i, h, lp, 0) - (intptr_t)P.k);
        vs = (long long)((intptr_t)snap_ptr(P, i, h, lp, 1) - (intptr_t)P.v);
      } else {
        ks = vs = (long long)pool_off(P, old_pg, h);
      }
    }
    s_ksrc[t] = ks;
    s_vsrc[t] = vs;
    if (lp < dp_hi) s_doff[t] = (long long)pool_off(P, new_pg, h);
  }
  const int lqpp = P.log_qpp, qpp = 1 << lqpp;  // 16-byte pieces per page
  const int lkq = P.log_kq;
  const int krow = D * es;
  for (int w0 = dp_lo; w0 < dp_hi; w0 += W) {
    const int w1 = min(w0 + W, dp_hi);          // destination pages [w0, w1)
    const int nsrc = w1 - w0 + P.span;          // source pages [w0, w1 + span - 1]
    const int nslots = (w1 - w0) << lb;
    lds_barrier();  // tables are set; the previous window is done with LDS
    for (int q = threadIdx.x; q < nslots; q += CP_THREADS) {
      const int j = (w0 << lb) + q;
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < MAX_EVICT; ++k) cnt += s_thr[k] <= j ? 1 : 0;
      s_src[q] = q + cnt;  // source slot relative to the window
    }
    lds_barrier();
    // every read of the window is issued before any is used, with no branch between them (a
    // piece past the window or the old pages reads a valid stand-in address and is discarded)
    const int nv = nsrc << lqpp;
    u32x4_t vreg[V_PIECES];
#pragma unroll
    for (int it = 0; it < V_PIECES; ++it) {
      const int q = threadIdx.x + it * CP_THREADS;
      const long long base = s_vsrc[w0 - dp_lo + min(q >> lqpp, nsrc - 1)];
      const long long o = (q < nv && base != NO_SRC) ? base + (long long)(q & (qpp - 1)) * 16 : 0;
      vreg[it] = *reinterpret_cast<const u32x4_t*>(P.v + o);
    }
    const int nk = nslots << lkq;
    u32x4_t kreg[K_PIECES];
#pragma unroll
    for (int it = 0; it < K_PIECES; ++it) {
      const int q = min((int)threadIdx.x + it * CP_THREADS, nk - 1);
      const int slot = q >> lkq, piece = q & ((1 << lkq) - 1);
      const int src = (w0 << lb) + s_src[slot];
      const long long base = s_ksrc[(src >> lb) - dp_lo];
      const long long o = base != NO_SRC ? base + (long long)(src & (b - 1)) * krow + piece * 16 : 0;
      kreg[it] = *reinterpret_cast<const u32x4_t*>(P.k + o);
    }
#pragma unroll
    for (int it = 0; it < V_PIECES; ++it) {
      const int q = threadIdx.x + it * CP_THREADS;
      if (q < nv) {
        const bool ok = s_vsrc[w0 - dp_lo + (q >> lqpp)] != NO_SRC;
        reinterpret_cast<u32x4_t*>(s_v)[q] = ok ? vreg[it] : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
    lds_barrier();  // every read of this window's sources precedes any write
#pragma unroll
    for (int it = 0; it < K_PIECES; ++it) {
      const int q = threadIdx.x + it * CP_THREADS;
      if (q < nk) {
        const int slot = q >> lkq, piece = q & ((1 << lkq) - 1);
        const int dp = w0 + (slot >> lb);
        reinterpret_cast<u32x4_t*>(P.k + s_doff[dp - dp_lo] + (size_t)(slot & (b - 1)) * krow)[piece] = kreg[it];
      }
    }
    // values: each lane writes two adjacent tokens of destination value rows, so the lanes of a
    // wave read consecutive tokens of a few rows from LDS (no bank conflicts) and write whole
    // 32- or 64-byte row segments. A lane keeps its token pair for the whole window: the pair's
    // two source slots are read once per destination page and serve all of its rows.
    const int lhb = lb - 1;                  // token pairs per row: 1 << lhb
    const int tp = threadIdx.x & ((1 << lhb) - 1), r0 = threadIdx.x >> lhb;
    const int rpi = CP_THREADS >> lhb;       // rows per pass of the block (32 or 16; D is a multiple)
    const size_t rb = (size_t)b * es;        // bytes of one value row
    for (int dpl = 0; dpl < w1 - w0; ++dpl) {
      const int slot = (dpl << lb) + 2 * tp;
      const int rs0 = s_src[slot], rs1 = s_src[slot + 1];
      const uint8_t* a0 = s_v + (size_t)(rs0 >> lb) * pb + (size_t)(rs0 & (b - 1)) * es;
      const uint8_t* a1 = s_v + (size_t)(rs1 >> lb) * pb + (size_t)(rs1 & (b - 1)) * es;
      uint8_t* dst = P.v + s_doff[w0 + dpl - dp_lo] + (size_t)(2 * tp) * es;
#pragma unroll 4
      for (int dd = r0; dd < D; dd += rpi) {
        if (es == 2) {
          const uint32_t x0 = *reinterpret_cast<const uint16_t*>(a0 + dd * rb);
          const uint32_t x1 = *reinterpret_cast<const uint16_t*>(a1 + dd * rb);
          *reinterpret_cast<uint32_t*>(dst + dd * rb) = x0 | (x1 << 16);
        } else {
          *reinterpret_cast<u32x2_t*>(dst + dd * rb) =
              u32x2_t{*reinterpret_cast<const uint32_t*>(a0 + dd * rb),
                      *reinterpret_cast<const uint32_t*>(a1 + dd * rb)};
        }
      }
    }
  }
  }
}

// Compaction for pages of 64..256 tokens. An item is (request, head, chunk, part); part p owns
// bytes [64p, 64p + 64) of every key row and the value rows [p Dp, (p + 1) Dp) (Dp = 64 bytes of
// elements), so items of different parts never touch the same bytes. The item rewrites its
// chunk's destination pages one at a time, left to right: destination page dp reads source
// pages dp .. dp + span, whose value rows of the part stay in an LDS ring of span + 1 slices
// (each source slice is fetched once), and key pieces go through registers, fetched one page
// ahead. A destination page overwrites only its own source page, which no later page of the
// item reads; the first `span` pages of the next chunk come from the snapshot.
constexpr int WIDE_KQ = 4;  // key pieces per thread and page: 256 slots x 4 pieces / CP_THREADS
constexpr int WIDE_VQ = 4;  // value pieces per thread and page slice
__global__ __launch_bounds__(CP_THREADS) void compact_wide_kernel(CParams P) {
  const int n_items = gp::uni(*P.n_items);
  const int L = P.chunk_pages, span = P.span, ring = span + 1, es = P.es;
  const int lb = P.log_b, b = 1 << lb;
  const int krow = P.D * es;
  const int vslice = WIDE_PART * b;         // bytes of one page's value rows of a part
  const int per = 16 / es;                  // elements per 16-byte piece
  __shared__ int s_thr[WIDE_MAX_EVICT];
  __shared__ int s_src[2 * 256];            // source slots of two destination pages' slots
  // source pages: byte offsets of the (page, head) blocks from the key and value pool bases (pool
  // or snapshot; NO_SRC past the old pages); destination pages: pool byte offsets
  __shared__ long long s_ksrc[CHUNK_PAGES + MAX_SPAN], s_vsrc[CHUNK_PAGES + MAX_SPAN];
  __shared__ long long s_doff[CHUNK_PAGES];
  extern __shared__ __align__(16) uint8_t s_ring[];  // ring x vslice bytes
  // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, and the parts of one
  // (request, head, chunk) read the two halves of the same 128-byte key lines, so all parts of a
  // chunk go to workgroups of one XCD (its L2 then serves the second half). Workgroup b of XCD
  // b % 8 takes the m-th part-item of the chunks g = b % 8 (mod 8), m = b / 8, b / 8 + S, ...
  const int n_groups = n_items / P.npart;
  const int xcd = blockIdx.x % NUM_XCD, S = gridDim.x / NUM_XCD;
  for (int m = blockIdx.x / NUM_XCD;; m += S) {
    const int g = xcd + NUM_XCD * (m / P.npart);
    if (g >= n_groups) break;
    const int item_k = g * P.npart + m % P.npart;
    lds_barrier();  // the previous item is done with the tables and the ring
    const int4 item = item_of(P, item_k);
    const int i = item.x / P.H_kv, h = item.x % P.H_kv;
    const int c = item.y / P.npart, part = item.y % P.npart;
    const Info inf = info_of(P, i);
    const int E = inf.E;
    const int dp0 = gp::uni(P.dp0[item.x]);
    const int dp_lo = max(dp0, c * L), dp_hi = min((c + 1) * L, inf.n_dest);
    for (int k = threadIdx.x; k < WIDE_MAX_EVICT; k += CP_THREADS)
      s_thr[k] = k < E ? P.ev[((size_t)i * P.H_kv + h) * P.max_evict + k] - k : INT_MAX;
    if (threadIdx.x < dp_hi - dp_lo + span) {
      const int lp = dp_lo + threadIdx.x;
      long long ks = NO_SRC, vs = NO_SRC;
      if (lp < inf.P) {
        if (from_snapshot(P, lp, c, inf)) {
          ks = (long long)((intptr_t)snap_ptr(P, i, h, lp, 0) - (intptr_t)P.k);
          vs = (long long)((intptr_t)snap_ptr(P, i, h, lp, 1) - (intptr_t)P.v);
        } else {
          ks = vs = (long long)pool_off(P, P.old_bt[(size_t)i * P.max_pages + lp], h);
        }
      }
      s_ksrc[threadIdx.x] = ks;
      s_vsrc[threadIdx.x] = vs;
      if (lp < dp_hi) s_doff[threadIdx.x] = (long long)pool_off(P, P.block_tables[(size_t)inf.r * P.max_pages + lp], h);
    }
    lds_barrier();
    const size_t koff = (size_t)part * WIDE_PART;  // the part's bytes inside a key row
    const size_t voff = (size_t)part * vslice;     // the part's value rows inside a page
    const int nk = b * (WIDE_PART / 16);
    // value rows of source page lp into registers, with no branch around the loads (a page past
    // the old pages, never read, takes a stand-in address and is zeroed when stored)
    auto load_slice = [&](int lp, u32x4_t (&r)[WIDE_VQ]) {
      const long long vs = s_vsrc[lp - dp_lo];
      const long long o = vs != NO_SRC ? vs + (long long)voff : 0;
#pragma unroll
      for (int it = 0; it < WIDE_VQ; ++it) {
        const int q = min((int)threadIdx.x + it * CP_THREADS, vslice / 16 - 1);
        r[it] = reinterpret_cast<const u32x4_t*>(P.v + o)[q];
      }
    };
    auto store_slice = [&](int lp, const u32x4_t (&r)[WIDE_VQ]) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(s_ring + (size_t)(lp % ring) * vslice);
      const bool have = s_vsrc[lp - dp_lo] != NO_SRC;
#pragma unroll
      for (int it = 0; it < WIDE_VQ; ++it) {
        const int q = threadIdx.x + it * CP_THREADS;
        if (q < vslice / 16) dst[q] = have ? r[it] : u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    // source slot of every destination slot of page dp, into table t: j + #{k : thr[k] <= j}
    // (thr is nondecreasing: a binary search)
    auto make_src = [&](int dp, int t) {
      for (int q = threadIdx.x; q < b; q += CP_THREADS) {
        const int j = (dp << lb) + q;
        int lo = 0, hi = E;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_thr[mid] <= j) lo = mid + 1;
          else hi = mid;
        }
        s_src[t * 256 + q] = j + lo;
      }
    };
    auto load_keys = [&](int t, u32x4_t (&kr)[WIDE_KQ]) {
#pragma unroll
      for (int it = 0; it < WIDE_KQ; ++it) {
        const int q = min((int)threadIdx.x + it * CP_THREADS, nk - 1);
        const int src = s_src[t * 256 + (q >> 2)];
        const long long ks = s_ksrc[(src >> lb) - dp_lo];
        const long long o = ks != NO_SRC ? ks + (long long)(src & (b - 1)) * krow + (long long)koff + (q & 3) * 16 : 0;
        kr[it] = *reinterpret_cast<const u32x4_t*>(P.k + o);
      }
    };
    // Software pipeline: while destination page dp is written, the key pieces of page dp + 1
    // and the value slice of page dp + 1 + span are already in flight. Those loads read pages
    // above dp only, which this item has not written yet.
    {
      u32x4_t r0[WIDE_VQ];
      for (int lp = dp_lo; lp < dp_lo + span; ++lp) {
        load_slice(lp, r0);
        store_slice(lp, r0);
      }
    }
    make_src(dp_lo, 0);
    lds_barrier();
    u32x4_t kA[WIDE_KQ], vA[WIDE_VQ];
    load_keys(0, kA);
    load_slice(dp_lo + span, vA);
    for (int dp = dp_lo; dp < dp_hi; ++dp) {
      const int t = (dp - dp_lo) & 1;
      // kA: key pieces of page dp; vA: value slice of source page dp + span
      store_slice(dp + span, vA);  // its ring slot held page dp - 1, which is finished
      const bool next = dp + 1 < dp_hi;
      if (next) make_src(dp + 1, t ^ 1);
      lds_barrier();  // slice dp + span and the next source table are visible
      u32x4_t kB[WIDE_KQ] = {}, vB[WIDE_VQ] = {};
      if (next) {
        load_keys(t ^ 1, kB);
        load_slice(dp + 1 + span, vB);
      }
      uint8_t* kd = P.k + s_doff[dp - dp_lo] + koff;
#pragma unroll
      for (int it = 0; it < WIDE_KQ; ++it) {
        const int q = threadIdx.x + it * CP_THREADS;
        if (q < nk) *reinterpret_cast<u32x4_t*>(kd + (size_t)(q >> 2) * krow + (q & 3) * 16) = kA[it];
      }
      // value rows: 16-byte pieces of destination rows gathered from the ring
      uint8_t* vd = P.v + s_doff[dp - dp_lo] + voff;
      const int lrp = lb + (es == 4 ? 2 : 1) - 4;  // log2 of the 16-byte pieces of a value row
      const int nvp = vslice / 16;
      for (int q = threadIdx.x; q < nvp; q += CP_THREADS) {
        const int dl = q >> lrp, piece = q & ((1 << lrp) - 1);
        uint32_t wv[4] = {0u, 0u, 0u, 0u};
        for (int e = 0; e < per; ++e) {
          const int rs = s_src[t * 256 + piece * per + e];
          const uint8_t* sp = s_ring + (size_t)((rs >> lb) % ring) * vslice +
                              ((size_t)dl * b + (rs & (b - 1))) * es;
          if (es == 2) wv[e >> 1] |= (uint32_t)(*reinterpret_cast<const uint16_t*>(sp)) << (16 * (e & 1));
          else wv[e] = *reinterpret_cast<const uint32_t*>(sp);
        }
        *reinterpret_cast<u32x4_t*>(vd + (size_t)q * 16) = u32x4_t{wv[0], wv[1], wv[2], wv[3]};
      }
      lds_barrier();  // every read of this page's ring slots precedes the next page's store
#pragma unroll
      for (int it = 0; it < WIDE_KQ; ++it) kA[it] = kB[it];
#pragma unroll
      for (int it = 0; it < WIDE_VQ; ++it) vA[it] = vB[it];
    }
  }
}

// ------------------------------------------------------------------ mixed-precision pages
// bf16 bits of a double, to nearest with ties to even: round to float with round-to-odd (the
// float keeps 16 more bits than bf16, also among subnormals), then float to bf16 to nearest even
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const float f = (float)x;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != x) {
    if (fabs(back) > fabs(x)) u -= 1u;  // the float rounded away from zero: step back
    u |= 1u;                            // inexact: odd
  }
  return gp::f32_to_bf16_bits(__uint_as_float(u));
}

// Destination tags of a compacting request (one workgroup per request): every head rewrites
// from the first destination page that changes for any head; a destination page keeps the
// precision of the pages that supply its tokens (any head) when they share one tag, else it
// becomes a bf16 page. Destination slot j takes source slot j + cnt(j), cnt(j) = #{k : ev[k] - k
// <= j}, an increasing map onto the kept tokens; so the sources of page dp in one head are the
// kept tokens between the sources of its first and last slots. The pages holding those two are
// suppliers; a page strictly between them (a shift of at most two pages leaves at most one)
// supplies iff not all of its b tokens are evicted. One thread per destination page; the heads'
// thresholds ev[k] - k sit in LDS, up to PLAN_HEADS heads at a time.
constexpr int PLAN_HEADS = 64;
constexpr int PLAN_THREADS = 256;  // destination pages per workgroup (grid: page blocks x requests)
__global__ __launch_bounds__(PLAN_THREADS) void mixed_plan_kernel(CParams P) {
  const int i = blockIdx.y;
  const Info inf = info_of(P, i);
  if (inf.mode != MODE_COMPACT) return;
  const int lb = P.log_b, b = 1 << lb, H = P.H_kv, E = inf.E;
  __shared__ int s_dpm;
  __shared__ __align__(16) int s_thr[PLAN_HEADS][MAX_EVICT];
  if (threadIdx.x == 0) {
    int m = INT_MAX;
    for (int h = 0; h < H; ++h) m = min(m, P.dp0[(size_t)i * H + h]);
    s_dpm = m;
  }
  __syncthreads();
  // (a workgroup of another block may already have lowered some heads' dp0 to this minimum:
  // the minimum is the same)
  const int dpm = gp::uni(s_dpm);
  if (blockIdx.x == 0)
    for (int h = threadIdx.x; h < H; h += blockDim.x) P.dp0[(size_t)i * H + h] = dpm;
  const int base = dpm + (int)blockIdx.x * PLAN_THREADS;
  if (base >= inf.n_dest) return;
  const int dp = base + (int)threadIdx.x;
  const bool mine = dp < inf.n_dest;
  // the tags of the three old pages that can supply page dp, fetched first
  int tag3[3];
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    const int lp = min(dp + s, inf.P - 1);
    tag3[s] = mine ? P.page_tag[P.old_bt[(size_t)i * P.max_pages + lp]] : GP_TAG_BF16;
  }
  const int j0 = dp << lb, j1 = j0 + b - 1;
  uint32_t supply = 0;
  for (int h0 = 0; h0 < H; h0 += PLAN_HEADS) {
    const int nh = min(PLAN_HEADS, H - h0);
    __syncthreads();  // the previous heads' thresholds are no longer read
    for (int e = threadIdx.x; e < nh * MAX_EVICT; e += blockDim.x) {
      const int hh = e / MAX_EVICT, k = e % MAX_EVICT;
      s_thr[hh][k] = k < E ? P.ev[((size_t)i * H + h0 + hh) * P.max_evict + k] - k : INT_MAX;
    }
    __syncthreads();
    if (!mine) continue;
    for (int hh = 0; hh < nh; ++hh) {
      const int4* th = reinterpret_cast<const int4*>(s_thr[hh]);
      int c0 = 0, c1 = 0;
#pragma unroll
      for (int k = 0; k < MAX_EVICT / 4; ++k) {
        const int4 t = th[k];
        c0 += (t.x <= j0) + (t.y <= j0) + (t.z <= j0) + (t.w <= j0);
        c1 += (t.x <= j1) + (t.y <= j1) + (t.z <= j1) + (t.w <= j1);
      }
      const int s_lo = ((j0 + c0) >> lb) - dp, s_hi = ((j1 + c1) >> lb) - dp;
      supply |= 1u << s_lo;
      supply |= 1u << s_hi;
      for (int s = s_lo + 1; s < s_hi; ++s) {
        // evictions inside old page dp + s: ev[k] = thr[k] + k in [lo, lo + b)
        const int lo = (dp + s) << lb;
        int ne = 0;
#pragma unroll
        for (int k = 0; k < MAX_EVICT / 4; ++k) {
          const int4 t = th[k];
          const int e0 = 4 * k;
          ne += (t.x != INT_MAX && t.x + e0 >= lo && t.x + e0 < lo + b);
          ne += (t.y != INT_MAX && t.y + e0 + 1 >= lo && t.y + e0 + 1 < lo + b);
          ne += (t.z != INT_MAX && t.z + e0 + 2 >= lo && t.z + e0 + 2 < lo + b);
          ne += (t.w != INT_MAX && t.w + e0 + 3 >= lo && t.w + e0 + 3 < lo + b);
        }
        if (ne < b) supply |= 1u << s;
      }
    }
  }
  if (!mine) return;
  // at most MAX_EVICT <= 2b evictions: a destination slot's source is at most two pages on
  int tag = -1;
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (!(supply >> s & 1u)) continue;
    tag = (tag < 0 || tag == tag3[s]) ? tag3[s] : GP_TAG_BF16;
  }
  P.new_tag[(size_t)i * P.max_pages + dp] = tag;
}

// The destination tags, written once every page of the call has moved.
__global__ __launch_bounds__(256) void mixed_tags_kernel(CParams P) {
  const int i = blockIdx.x;
  const Info inf = info_of(P, i);
  if (inf.mode != MODE_COMPACT) return;
  const int dpm = P.dp0[(size_t)i * P.H_kv];
  for (int dp = dpm + (int)threadIdx.x; dp < inf.n_dest; dp += blockDim.x)
    P.page_tag[P.block_tables[(size_t)inf.r * P.max_pages + dp]] =
        (uint8_t)P.new_tag[(size_t)i * P.max_pages + dp];
}

// Bytes of one (page, KV head) in a format: key part and value part (codes, then the row
// scales); the snapshot and the LDS staging hold a page in its own format this way.
struct MixedBytes {
  int kc, vc, sc;  // key code bytes, value code bytes, scale bytes per part
};
__device__ __forceinline__ MixedBytes mixed_bytes(int tag, int b, int D) {
  if (tag == GP_TAG_FP8) return MixedBytes{b * D, b * D, 4 * b};
  if (tag == GP_TAG_INT4) return MixedBytes{b * D / 2, b * D / 2, 2 * b};
  return MixedBytes{2 * b * D, 2 * b * D, 0};
}
// (page, head) sources of each part in the pools
__device__ __forceinline__ void mixed_src(const CParams& P, int tag, int pg, int h, const uint8_t** kc,
                                          const uint8_t** vc, const uint8_t** ks, const uint8_t** vs) {
  const size_t ph = (size_t)pg * P.H_kv + h, b = P.page_size, D = P.D;
  if (tag == GP_TAG_FP8) {
    *kc = P.k8 + ph * b * D;
    *vc = P.v8 + ph * b * D;
    *ks = reinterpret_cast<const uint8_t*>(P.k_scale + ph * b);
    *vs = reinterpret_cast<const uint8_t*>(P.v_scale + ph * b);
  } else if (tag == GP_TAG_INT4) {
    *kc = P.k4 + ph * b * D / 2;
    *vc = P.v4 + ph * b * D / 2;
    *ks = reinterpret_cast<const uint8_t*>(P.k4_scale + ph * b);
    *vs = reinterpret_cast<const uint8_t*>(P.v4_scale + ph * b);
  } else {
    *kc = P.k + ph * b * D * 2;
    *vc = P.v + ph * b * D * 2;
    *ks = *vs = nullptr;
  }
}

// One (page, head) block of a mixed cache in registers: this thread's pieces of the key and
// value codes (at most 2 x CP_THREADS 16-byte pieces each: a 32-token bf16 page) and of the two
// row-scale vectors (at most CP_THREADS words). Every load is issued before any is used; a
// thread past a part's end reads the part's last piece again (or the key codes for a page
// without scales) and stores nothing.
struct PageParts {
  u32x4_t k[2], v[2];
  uint32_t ks, vs;
};
__device__ __forceinline__ PageParts load_page_parts(const uint8_t* kc, const uint8_t* vc,
                                                     const uint8_t* ks, const uint8_t* vs,
                                                     const MixedBytes& mb) {
  const int t = threadIdx.x, nc = mb.kc / 16, ns = mb.sc / 4;
  const u32x4_t* k16 = reinterpret_cast<const u32x4_t*>(kc);
  const u32x4_t* v16 = reinterpret_cast<const u32x4_t*>(vc);
  const uint32_t* k4 = reinterpret_cast<const uint32_t*>(ns ? ks : kc);
  const uint32_t* v4 = reinterpret_cast<const uint32_t*>(ns ? vs : vc);
  PageParts x;
  x.k[0] = k16[min(t, nc - 1)];
  x.k[1] = k16[min(t + CP_THREADS, nc - 1)];
  x.v[0] = v16[min(t, nc - 1)];
  x.v[1] = v16[min(t + CP_THREADS, nc - 1)];
  x.ks = k4[min(t, max(ns, 1) - 1)];
  x.vs = v4[min(t, max(ns, 1) - 1)];
  return x;
}
__device__ __forceinline__ void store_page_parts(const PageParts& x, uint8_t* kd, uint8_t* vd,
                                                 uint8_t* ksd, uint8_t* vsd, const MixedBytes& mb) {
  const int t = threadIdx.x, nc = mb.kc / 16, ns = mb.sc / 4;
  if (t < nc) {
    reinterpret_cast<u32x4_t*>(kd)[t] = x.k[0];
    reinterpret_cast<u32x4_t*>(vd)[t] = x.v[0];
  }
  if (t + CP_THREADS < nc) {
    reinterpret_cast<u32x4_t*>(kd)[t + CP_THREADS] = x.k[1];
    reinterpret_cast<u32x4_t*>(vd)[t + CP_THREADS] = x.v[1];
  }
  if (t < ns) {
    reinterpret_cast<uint32_t*>(ksd)[t] = x.ks;
    reinterpret_cast<uint32_t*>(vsd)[t] = x.vs;
  }
}

// The snapshot of a mixed cache holds the saved page in its own format.
__global__ __launch_bounds__(CP_THREADS) void snapshot_mixed_kernel(CParams P) {
  const int n_items = gp::uni(*P.n_items);
  for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int4 item = item_of(P, it);
    const int i = item.x / P.H_kv, h = item.x % P.H_kv, c = item.y;
    const Info inf = info_of(P, i);
    for (int s = 0; s < P.span; ++s) {
      const int lp = (c + 1) * P.chunk_pages + s;
      if (!from_snapshot(P, lp, c, inf)) continue;
      const int pg = P.old_bt[(size_t)i * P.max_pages + lp];
      const int tag = P.page_tag[pg];
      const MixedBytes mb = mixed_bytes(tag, P.page_size, P.D);
      const uint8_t *kc, *vc, *ks, *vs;
      mixed_src(P, tag, pg, h, &kc, &vc, &ks, &vs);
      uint8_t* kd = snap_ptr(P, i, h, lp, 0);
      uint8_t* vd = snap_ptr(P, i, h, lp, 1);
      const PageParts x = load_page_parts(kc, vc, ks, vs, mb);
      store_page_parts(x, kd, vd, kd + mb.kc, vd + mb.vc, mb);
    }
  }
}

// signed nibble n (0..7 from the low end) of a 32-bit word
__device__ __forceinline__ int nib(uint32_t w, int n) { return (int32_t)(w << (28 - 4 * n)) >> 28; }

// Compaction of a mixed-precision cache (pages of 16 or 32 tokens), in windows of W destination
// pages like the uniform path. Per window the source slot of every destination slot is tabulated;
// the value parts (codes, then row scales) of the W + span source pages are staged in LDS in
// their own formats, since a value row gathers one element per token; every key piece of the
// window is read into registers straight from its source row. The destination page is written in
// its new format: the same format as every source (codes and row scales copied; INT4 value
// nibbles regrouped into four-token blocks) or bf16 (each element's exact code * scale rounded
// once). All loads of a window are issued before any is used, at valid stand-in addresses where a
// piece has no source. Every source and destination block is a byte offset from the bf16 key
// pool's base, which keeps the accesses in the global address space. The ordering argument of
// compact_kernel holds unchanged: a window reads only pages at or above its own destination
// pages (the next chunk's first pages from the snapshot), and every staged byte is read before
// the barrier that precedes the next window's staging.
constexpr int MXK_PIECES = 4;   // key pieces per thread and window (16-byte pieces of bf16 rows)
constexpr int MXV_PIECES = 8;   // staged value pieces per thread and window
__device__ __forceinline__ int mx_row_bytes(int tag, int D) {
  return tag == GP_TAG_FP8 ? D : (tag == GP_TAG_INT4 ? D / 2 : 2 * D);
}
__device__ __forceinline__ int mx_scale_bytes(int tag) {
  return tag == GP_TAG_FP8 ? 4 : (tag == GP_TAG_INT4 ? 2 : 0);
}
// word w (0..3) of a 16-byte piece
__device__ __forceinline__ uint32_t word_of(const u32x4_t& x, int w) {
  return w == 0 ? x[0] : (w == 1 ? x[1] : (w == 2 ? x[2] : x[3]));
}
// bf16 bits of a * b rounded once, to nearest with ties to even. The float product can only go
// wrong when it lands exactly on a bf16 midpoint while the exact product does not: its residual
// (an fma, exact for a normal product of normal factors) then says which way to round. Zero
// products are exact; nonzero ones below 2^-96, or a subnormal b, take the float64 route.
__device__ __forceinline__ uint32_t mul_to_bf16_bits(float a, float b) {
  const float p = a * b;
  if ((fabsf(p) < 0x1p-96f && p != 0.f) || fabsf(b) < 0x1p-126f)
    return f64_to_bf16_bits((double)a * (double)b);
  const uint32_t u = __float_as_uint(p);
  if ((u & 0xffffu) == 0x8000u) {
    const float e = __builtin_fmaf(a, b, -p);
    if (e != 0.f) return (u >> 16) + (((__float_as_uint(e) ^ u) >> 31) ^ 1u);
  }
  return gp::f32_to_bf16_bits(p);
}
// bf16 bits of the element with fp8 code c (low byte) times an fp32 row scale: one rounding
__device__ __forceinline__ uint32_t fp8_times(uint32_t c, float sc) {
  return mul_to_bf16_bits(__builtin_amdgcn_cvt_pk_f32_fp8(c, false)[0], sc);
}
// bf16 bits of INT4 code q times a half row scale: the product is exact in float
__device__ __forceinline__ uint32_t int4_times(int q, float sc) {
  return gp::f32_to_bf16_bits((float)q * sc);
}
typedef __bf16 mx_bf16x2 __attribute__((ext_vector_type(2)));
typedef float mx_f32x2 __attribute__((ext_vector_type(2)));
// two floats to a bf16 pair (low half p0), to nearest even, in one instruction on gfx950
__device__ __forceinline__ uint32_t pk_bf16(float p0, float p1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((mx_f32x2){p0, p1}, mx_bf16x2));
}
// The products x0 * s0 and x1 * s1 rounded once to a bf16 pair, where each x is exact in float
// and each product either exact in float (INT4 codes times a half scale) or an fp8 value times a
// float scale of magnitude in [2^-87, 2^100) (a normal product whose float rounding is off by at
// most half a float ulp). The hardware rounding of the float product is then right unless that
// product sits exactly on a bf16 midpoint while the exact one does not: the product's fma residual
// (exact for a normal product) gives the side. `inexact` marks the products that may have rounded.
__device__ __forceinline__ uint32_t pair_to_bf16(float x0, float s0, bool inexact0, float x1, float s1,
                                                 bool inexact1) {
  const float p0 = x0 * s0, p1 = x1 * s1;
  uint32_t r = pk_bf16(p0, p1);
  const uint32_t u0 = __float_as_uint(p0), u1 = __float_as_uint(p1);
  const bool m0 = inexact0 && (u0 & 0xffffu) == 0x8000u, m1 = inexact1 && (u1 & 0xffffu) == 0x8000u;
  if (__builtin_expect(m0 || m1, 0)) {
    const float e0 = __builtin_fmaf(x0, s0, -p0), e1 = __builtin_fmaf(x1, s1, -p1);
    if (m0 && e0 != 0.f) r = (r & 0xffff0000u) | ((u0 >> 16) + (((__float_as_uint(e0) ^ u0) >> 31) ^ 1u));
    if (m1 && e1 != 0.f) r = (r & 0xffffu) | (((u1 >> 16) + (((__float_as_uint(e1) ^ u1) >> 31) ^ 1u)) << 16);
  }
  return r;
}
// a float scale that keeps every nonzero fp8 product normal (fp8 values are at least 2^-9)
__device__ __forceinline__ bool fp8_scale_fast(float sc) { return fabsf(sc) >= 0x1p-87f && fabsf(sc) < 0x1p100f; }
__device__ __forceinline__ float half_bits_to_f32(uint32_t hs) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)hs);
}
__global__ __launch_bounds__(CP_THREADS) void compact_mixed_kernel(CParams P) {
  const int n_items = gp::uni(*P.n_items);
  const int L = P.chunk_pages, W = P.window_pages, span = P.span;
  const int lb = P.log_b, b = 1 << lb, D = P.D;
  const int VS = 2 * b * D;                 // LDS slot of one source value part (bf16 codes is the largest)
  const int lnpv = lb + __builtin_ctz(D) - 3;   // log2 of the 16-byte pieces of a slot
  const int lnpr = __builtin_ctz(D) - 3;        // log2 of the 16-byte pieces of a bf16 key row
  const int vslot = D / 16;                 // INT4 value dimension slot: (e % 16) * (D/16) + e / 16
  extern __shared__ __align__(16) uint8_t s_v[];  // (W + span) slots of VS bytes
  __shared__ int s_thr[MAX_EVICT];
  __shared__ int s_src[MAX_WINDOW_SLOTS];
  __shared__ int s_stag[CHUNK_PAGES + MAX_SPAN], s_dtag[CHUNK_PAGES];
  __shared__ long long s_kc[CHUNK_PAGES + MAX_SPAN], s_ks[CHUNK_PAGES + MAX_SPAN];
  __shared__ long long s_vc[CHUNK_PAGES + MAX_SPAN], s_vs[CHUNK_PAGES + MAX_SPAN];
  __shared__ long long s_dk[CHUNK_PAGES], s_dks[CHUNK_PAGES], s_dv[CHUNK_PAGES], s_dvs[CHUNK_PAGES];
  uint8_t* const base = P.k;
  auto off = [&](const void* p) { return (long long)((intptr_t)p - (intptr_t)base); };
  // stand-in pieces: 16 * (q & sm) stays inside the bf16 key pool (at most its first 16 KB)
  const long long pool_pieces = (long long)P.num_pages * P.H_kv * b * D * 2 / 16;
  const int sm = (int)(1ll << (63 - __builtin_clzll((unsigned long long)min(pool_pieces, 1024ll)))) - 1;
  for (int item_k = blockIdx.x; item_k < n_items; item_k += gridDim.x) {
    lds_barrier();  // the previous item is done with the tables and LDS
    const int4 item = item_of(P, item_k);
    const int i = item.x / P.H_kv, h = item.x % P.H_kv, c = item.y;
    const Info inf = info_of(P, i);
    const int E = inf.E;
    const int dp0 = gp::uni(P.dp0[item.x]);
    const int dp_lo = max(dp0, c * L), dp_hi = min((c + 1) * L, inf.n_dest);
    if (threadIdx.x < MAX_EVICT)
      s_thr[threadIdx.x] = (int)threadIdx.x < E
                               ? P.ev[((size_t)i * P.H_kv + h) * P.max_evict + threadIdx.x] - (int)threadIdx.x
                               : INT_MAX;
    if (threadIdx.x < dp_hi - dp_lo + span) {
      const int t = threadIdx.x, lp = dp_lo + t;
      int tag = GP_TAG_BF16;
      long long kc = NO_SRC, ks = NO_SRC, vc = NO_SRC, vs = NO_SRC;
      if (lp < inf.P) {
        const int pg = P.old_bt[(size_t)i * P.max_pages + lp];
        tag = P.page_tag[pg];
        const MixedBytes mb = mixed_bytes(tag, b, D);
        const uint8_t *pk, *pv, *pks, *pvs;
        if (from_snapshot(P, lp, c, inf)) {
          pk = snap_ptr(P, i, h, lp, 0);
          pv = snap_ptr(P, i, h, lp, 1);
          pks = pk + mb.kc;
          pvs = pv + mb.vc;
        } else {
          mixed_src(P, tag, pg, h, &pk, &pv, &pks, &pvs);
        }
        kc = off(pk);
        vc = off(pv);
        ks = pks ? off(pks) : 0;
        vs = pvs ? off(pvs) : 0;
      }
      s_stag[t] = tag;
      s_kc[t] = kc;
      s_ks[t] = ks;
      s_vc[t] = vc;
      s_vs[t] = vs;
      if (lp < dp_hi) {
        const int td = P.new_tag[(size_t)i * P.max_pages + lp];
        const uint8_t *pk, *pv, *pks, *pvs;
        mixed_src(P, td, P.block_tables[(size_t)inf.r * P.max_pages + lp], h, &pk, &pv, &pks, &pvs);
        s_dtag[t] = td;
        s_dk[t] = off(pk);
        s_dv[t] = off(pv);
        s_dks[t] = pks ? off(pks) : 0;
        s_dvs[t] = pvs ? off(pvs) : 0;
      }
    }
    for (int w0 = dp_lo; w0 < dp_hi; w0 += W) {
      const int w1 = min(w0 + W, dp_hi);  // destination pages [w0, w1)
      const int nsrc = w1 - w0 + span;    // source pages [w0, w1 + span - 1]
      const int nslots = (w1 - w0) << lb;
      const int t0 = w0 - dp_lo;          // table index of page w0
      // the thread index, opaque to the compiler inside the window: otherwise it hoists every
      // per-piece index out of the loops and holds them in registers for the whole kernel
      int tx = threadIdx.x;
      asm volatile("" : "+v"(tx));
      lds_barrier();  // tables are set; the previous window is done with LDS
      for (int q = tx; q < nslots; q += CP_THREADS) {
        const int j = (w0 << lb) + q;
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < MAX_EVICT; ++k) cnt += s_thr[k] <= j ? 1 : 0;
        s_src[q] = q + cnt;  // source slot relative to the window
      }
      lds_barrier();
      // key pieces on the bf16 row grid: piece p of destination row `slot`, from the source row in
      // its own format (a converted piece reads 8 fp8 codes or 8 INT4 nibbles and the row scale)
      const int nk = nslots << lnpr;
      u32x4_t kreg[MXK_PIECES];
      uint32_t kscale[MXK_PIECES];
#pragma unroll
      for (int it = 0; it < MXK_PIECES; ++it) {
        const int q = min(tx + it * CP_THREADS, nk - 1);
        const int slot = q >> lnpr, p = q & ((1 << lnpr) - 1);
        const int td = s_dtag[t0 + (slot >> lb)];
        const int src = s_src[slot];
        const int ts = s_stag[t0 + (src >> lb)], so = src & (b - 1);
        const long long kc = s_kc[t0 + (src >> lb)];
        const int sub = ts == td ? 16 * p : (ts == GP_TAG_FP8 ? 8 * p : 4 * p);
        const bool ok = 16 * p < mx_row_bytes(td, D) && kc != NO_SRC;
        const long long row = kc != NO_SRC ? kc + (long long)so * mx_row_bytes(ts, D) : 16 * (q & sm);
        const long long o = ok ? row + (sub & ~15) : row;  // a piece past the row: the row's first
        kreg[it] = *reinterpret_cast<const u32x4_t*>(base + o);
        const long long so_s = (ok && ts != td) ? s_ks[t0 + (src >> lb)] + (long long)so * mx_scale_bytes(ts) : o;
        kscale[it] = *reinterpret_cast<const uint32_t*>(base + (so_s & ~3ll));
        kscale[it] = (so_s & 2) ? kscale[it] >> 16 : kscale[it];
      }
      // key row scale of destination row tx (fp8 / INT4 destinations; nslots <= threads)
      uint32_t ksrow;
      {
        const int q = min(tx, nslots - 1);
        const int td = s_dtag[t0 + (q >> lb)], src = s_src[q];
        const long long ks = s_ks[t0 + (src >> lb)], kc = s_kc[t0 + (src >> lb)];
        const long long so_s = (td != GP_TAG_BF16 && ks != NO_SRC)
                                   ? ks + (long long)(src & (b - 1)) * mx_scale_bytes(td)
                                   : (kc != NO_SRC ? kc : 16 * (q & sm));
        ksrow = *reinterpret_cast<const uint32_t*>(base + (so_s & ~3ll));
        ksrow = (so_s & 2) ? ksrow >> 16 : ksrow;
      }
      // value parts of the source pages, straight into LDS (one 16-byte piece per lane, a wave's
      // pieces contiguous): piece k of slot t is codes piece k, then the scale pieces; lanes with
      // no piece to stage issue no load
#pragma unroll
      for (int it = 0; it < MXV_PIECES; ++it) {
        const int q = tx + it * CP_THREADS;
        const int t = min(q >> lnpv, nsrc - 1), k = q & ((1 << lnpv) - 1);
        const MixedBytes mb = mixed_bytes(s_stag[t0 + t], b, D);
        const long long vc = s_vc[t0 + t];
        if (q >> lnpv < nsrc && vc != NO_SRC && 16 * k < mb.vc + mb.sc) {
          const long long o = 16 * k < mb.vc ? vc + 16 * k : s_vs[t0 + t] + (16 * k - mb.vc);
          __builtin_amdgcn_global_load_lds(
              static_cast<const void*>(base + o),
              (__attribute__((address_space(3))) void*)(s_v + 16 * ((tx & ~(GP_WAVE - 1)) + it * CP_THREADS)), 16, 0, 0);
        }
      }
      // every load of the window has landed (the staged pieces in LDS too) before any write
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int it = 0; it < MXK_PIECES; ++it) {
        const int q = tx + it * CP_THREADS;
        if (q >= nk) continue;
        const int slot = q >> lnpr, p = q & ((1 << lnpr) - 1);
        const int dpl = slot >> lb, td = s_dtag[t0 + dpl];
        if (16 * p >= mx_row_bytes(td, D)) continue;
        const int src = s_src[slot];
        const int ts = s_stag[t0 + (src >> lb)];
        const u32x4_t kr = kreg[it];
        const uint32_t ksc = kscale[it];
        u32x4_t out = kr;
        if (ts != td) {  // td is bf16: 8 elements 8p .. 8p + 7
          uint32_t e[4];
          if (ts == GP_TAG_FP8) {
            const int w = ((8 * p) & 15) >> 2;  // 0 or 2
            const uint32_t wd[2] = {word_of(kr, w), word_of(kr, w + 1)};
            const float sc = __uint_as_float(ksc);
            if (__builtin_expect(!fp8_scale_fast(sc), 0)) {
              // a scale outside the fast range: element by element, the exact route
              uint16_t* kd16 = reinterpret_cast<uint16_t*>(
                  base + s_dk[t0 + dpl] + (long long)(slot & (b - 1)) * mx_row_bytes(td, D) + 16 * p);
#pragma unroll 1
              for (int m = 0; m < 8; ++m) kd16[m] = (uint16_t)fp8_times(wd[m >> 2] >> (8 * (m & 3)), sc);
              continue;
            }
            const mx_f32x2 f[4] = {__builtin_amdgcn_cvt_pk_f32_fp8(wd[0], false), __builtin_amdgcn_cvt_pk_f32_fp8(wd[0], true),
                                   __builtin_amdgcn_cvt_pk_f32_fp8(wd[1], false), __builtin_amdgcn_cvt_pk_f32_fp8(wd[1], true)};
#pragma unroll
            for (int m = 0; m < 4; ++m) e[m] = pair_to_bf16(f[m][0], sc, true, f[m][1], sc, true);
          } else {
            const uint32_t wd = word_of(kr, ((4 * p) & 15) >> 2);
            const float sc = half_bits_to_f32(ksc & 0xffffu);
#pragma unroll
            for (int m = 0; m < 4; ++m) e[m] = pk_bf16((float)nib(wd, 2 * m) * sc, (float)nib(wd, 2 * m + 1) * sc);
          }
          out = u32x4_t{e[0], e[1], e[2], e[3]};
        }
        *reinterpret_cast<u32x4_t*>(base + s_dk[t0 + dpl] + (long long)(slot & (b - 1)) * mx_row_bytes(td, D) + 16 * p) = out;
        __builtin_amdgcn_sched_barrier(0);  // one piece's conversion at a time: fewer live registers
      }
      // row scales of fp8 / INT4 destination rows (every source of such a page has its format):
      // the key scale read above, the value scale from the staged slot
      if (tx < nslots) {
        const int q = tx, dpl = q >> lb, td = s_dtag[t0 + dpl];
        if (td != GP_TAG_BF16) {
          const int src = s_src[q], so = src & (b - 1), row = q & (b - 1);
          const uint8_t* vsc = s_v + (size_t)(src >> lb) * VS + mixed_bytes(td, b, D).vc;
          if (td == GP_TAG_FP8) {
            reinterpret_cast<uint32_t*>(base + s_dks[t0 + dpl])[row] = ksrow;
            reinterpret_cast<uint32_t*>(base + s_dvs[t0 + dpl])[row] = reinterpret_cast<const uint32_t*>(vsc)[so];
          } else {
            reinterpret_cast<uint16_t*>(base + s_dks[t0 + dpl])[row] = (uint16_t)ksrow;
            reinterpret_cast<uint16_t*>(base + s_dvs[t0 + dpl])[row] = reinterpret_cast<const uint16_t*>(vsc)[so];
          }
        }
      }
      // values, gathered from the staged slots. bf16 and fp8 destinations ([D][b] rows): a lane
      // takes two adjacent tokens, whose sources it looks up once per page, and writes them in
      // every row it owns; INT4 destinations ([b/4][D][2]): a lane writes the two bytes of one
      // dimension slot of a four-token block.
      const int lhb = lb - 1;
      const int tp = tx & ((1 << lhb) - 1), r0 = tx >> lhb;
      const int rpi = CP_THREADS >> lhb;
      for (int dpl = 0; dpl < w1 - w0; ++dpl) {
        const int td = s_dtag[t0 + dpl];
        uint8_t* dv = base + s_dv[t0 + dpl];
        if (td == GP_TAG_INT4) {
          for (int u = tx; u < (b >> 2) * D; u += CP_THREADS) {
            const int ds = u % D, Q = u / D;
            uint32_t out = 0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
              const int src = s_src[(dpl << lb) + 4 * Q + m], so = src & (b - 1);
              const uint8_t* a = s_v + (size_t)(src >> lb) * VS;
              const uint32_t byte = a[((so >> 2) * D + ds) * 2 + ((so & 3) >> 1)];
              out |= ((byte >> (4 * (so & 1))) & 0xFu) << (4 * m);
            }
            reinterpret_cast<uint16_t*>(dv)[Q * D + ds] = (uint16_t)out;
          }
          continue;
        }
        int so[2], tg[2];
        const uint8_t* a[2];
        float sc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int src = s_src[(dpl << lb) + 2 * tp + m];
          so[m] = src & (b - 1);
          tg[m] = s_stag[t0 + (src >> lb)];
          a[m] = s_v + (size_t)(src >> lb) * VS;
          const MixedBytes mb = mixed_bytes(tg[m], b, D);
          sc[m] = tg[m] == GP_TAG_FP8 ? reinterpret_cast<const float*>(a[m] + mb.vc)[so[m]]
                  : tg[m] == GP_TAG_INT4 ? half_bits_to_f32(reinterpret_cast<const uint16_t*>(a[m] + mb.vc)[so[m]])
                                         : 1.f;
        }
        if (td == GP_TAG_FP8) {
          #pragma unroll 4
          for (int dd = r0; dd < D; dd += rpi) {
            const uint32_t x0 = a[0][dd * b + so[0]], x1 = a[1][dd * b + so[1]];
            reinterpret_cast<uint16_t*>(dv + dd * b)[tp] = (uint16_t)(x0 | (x1 << 8));
          }
          continue;
        }
        // bf16 destination. fp8 tokens with a scale outside the fast range go element by
        // element the exact way; otherwise each row reads the 32-bit LDS word holding each
        // token's element (a bf16 half, an fp8 byte or an INT4 nibble's byte), takes the
        // element as a float times its scale (bf16 bits are kept as they are) and rounds the two
        // tokens with one packed conversion
        const bool slow = (tg[0] == GP_TAG_FP8 && !fp8_scale_fast(sc[0])) ||
                          (tg[1] == GP_TAG_FP8 && !fp8_scale_fast(sc[1]));
        if (__builtin_expect(slow, 0)) {
#pragma unroll 1
          for (int e = 0; e < 2 * (D / rpi); ++e) {
            const int m = e & 1, dd = r0 + (e >> 1) * rpi;
            uint32_t x;
            if (tg[m] == GP_TAG_BF16) {
              x = reinterpret_cast<const uint16_t*>(a[m])[dd * b + so[m]];
            } else if (tg[m] == GP_TAG_FP8) {
              x = fp8_times(a[m][dd * b + so[m]], sc[m]);
            } else {
              const int sl = (dd % 16) * vslot + dd / 16;
              x = int4_times(nib(a[m][((so[m] >> 2) * D + sl) * 2 + ((so[m] & 3) >> 1)], so[m] & 1), sc[m]);
            }
            reinterpret_cast<uint16_t*>(dv + dd * 2 * b)[2 * tp + m] = (uint16_t)x;
          }
          continue;
        }
        // a token's element of row r0 + k rpi sits at va + k vk bytes of its slot (rpi is a
        // multiple of 16, so the INT4 dimension slot steps by rpi / 16 as well); the address,
        // the conversion and the result are picked by arithmetic selects, so the rows of a page
        // carry no branch and their LDS reads go out together
        int va[2], vk[2];
        bool f8[2], bf[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f8[m] = tg[m] == GP_TAG_FP8;
          bf[m] = tg[m] == GP_TAG_BF16;
          const int a_bf = (so[m] + b * r0) * 2, a_f8 = so[m] + b * r0;
          const int a_i4 = ((so[m] >> 2) * D + (r0 % 16) * vslot + r0 / 16) * 2 + ((so[m] & 3) >> 1);
          va[m] = bf[m] ? a_bf : (f8[m] ? a_f8 : a_i4);
          vk[m] = bf[m] ? 2 * b * rpi : (f8[m] ? b * rpi : 2 * (rpi / 16));
        }
        const int nrow = D / rpi;  // 2, 4 or 8
        for (int k0 = 0; k0 < nrow; k0 += 4) {
          uint32_t y[4][2];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const int ad = va[m] + min(k0 + k, nrow - 1) * vk[m];
              y[k][m] = *reinterpret_cast<const uint32_t*>(a[m] + (ad & ~3)) >> ((ad & 3) * 8);
            }
          }
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (k0 + k >= nrow) continue;
            float f[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const uint32_t u8 = __float_as_uint(__builtin_amdgcn_cvt_pk_f32_fp8(y[k][m], false)[0]);
              const uint32_t u4 = __float_as_uint((float)nib(y[k][m], so[m] & 1));
              const uint32_t msk = 0u - (uint32_t)f8[m];
              f[m] = __uint_as_float((u8 & msk) | (u4 & ~msk));
            }
            const uint32_t cv = pair_to_bf16(f[0], sc[0], f8[0], f[1], sc[1], f8[1]);
            const uint32_t m0 = 0u - (uint32_t)bf[0], m1 = 0u - (uint32_t)bf[1];
            const uint32_t lo = ((y[k][0] & 0xffffu) & m0) | (cv & 0xffffu & ~m0);
            const uint32_t hi = ((y[k][1] << 16) & m1) | (cv & 0xffff0000u & ~m1);
            reinterpret_cast<uint32_t*>(dv + (r0 + (k0 + k) * rpi) * 2 * b)[tp] = lo | hi;
          }
        }
      }
    }
  }
}

// Window of a mixed-precision compaction: the W * b destination key rows (bf16-sized) must fit
// MXK_PIECES pieces per thread and the W + span staged value parts MXV_PIECES.
int mixed_window_pages(int page_size, int D, int span) {
  int W = 8;
  while (W > 1 && ((long)W * page_size * (D / 8) > (long)MXK_PIECES * CP_THREADS ||
                   (long)(W + span) * page_size * (D / 8) > (long)MXV_PIECES * CP_THREADS))
    --W;
  return W;
}

// Window of W destination pages: LDS holds the W + span source value pages, and the W * b key
// rows must fit K_PIECES 16-byte pieces per thread.
int window_pages_for(int page_size, int D, int es, int span) {
  const long pv = (long)page_size * D * es;
  int W = (int)(CP_LDS_BYTES / pv) - span;
  W = std::max(1, std::min(8, W));
  while (W > 1 && ((long)W * page_size * D * es > (long)K_PIECES * CP_THREADS * 16 ||
                   (long)(W + span) * page_size * D * es > (long)V_PIECES * CP_THREADS * 16))
    --W;
  return W;
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
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) ++l;
  return l;
}


}  // namespace

namespace {

// Workspace: per call the request records, old block-table rows and release list; per layer the
// evicted lists, first changed pages and chunk work list; shared by the layers (used one layer
// at a time, in stream order) the selection survivors and the chunk snapshots.
struct WsLayout {
  size_t info, old_bt, rel, new_tag, chk, layer0, layer_bytes, ev, dp0, items, n_items, cand, snap, total;
};

// destination pages per compaction item: the call's shape decides, so that the workspace size
// and the call agree
int chunk_pages_for(int R, int H_kv, int page_size, int C_max) {
  if (page_size >= WIDE_MIN_PAGE) return WIDE_CHUNK_PAGES;
  const long chunks16 = ((long)C_max / page_size + 1 + CHUNK_PAGES - 1) / CHUNK_PAGES;
  return (long)R * H_kv * chunks16 <= SMALL_CALL_ITEMS ? CHUNK_PAGES / 2 : CHUNK_PAGES;
}

WsLayout ws_layout(int L, int R, int H_kv, int max_pages, int page_size, int C_max) {
  // snapshots sized for the widest supported element (fp32) and head_dim 128
  const int es = 4, D = 128;
  const bool wide = page_size >= WIDE_MIN_PAGE;
  const size_t max_evict = wide ? 2 * (size_t)page_size : MAX_EVICT;
  const size_t parts = wide ? WIDE_MAX_PARTS : 1;
  const size_t cp = (size_t)chunk_pages_for(R, H_kv, page_size, C_max);
  const size_t max_chunks = (size_t)(max_pages + cp - 1) / cp;
  WsLayout w{};
  size_t off = 0;
  w.info = off;
  off += (size_t)R * sizeof(Info);
  w.old_bt = off;
  off += (size_t)R * max_pages * 4;
  w.rel = off;
  off += (size_t)R * max_pages * 4;
  w.new_tag = off;
  off += (size_t)R * max_pages * 4;
  w.chk = off;
  off += (size_t)R * 2 * 4;
  off = (off + 255) & ~(size_t)255;
  w.layer0 = off;
  w.ev = 0;
  size_t lo = (size_t)R * H_kv * max_evict * 4;
  w.dp0 = lo;
  lo += (size_t)R * H_kv * 4;
  lo = (lo + 15) & ~(size_t)15;
  w.items = lo;
  lo += (size_t)R * H_kv * max_chunks * parts * sizeof(int4);
  w.n_items = lo;
  lo += 256;
  w.layer_bytes = (lo + 255) & ~(size_t)255;
  off += (size_t)L * w.layer_bytes;
  w.cand = off;
  off += (size_t)R * H_kv * SEL_MAX_CHUNKS * MAX_EVICT * 8;
  w.snap = off;
  off += (size_t)R * H_kv * max_chunks * MAX_SPAN * 2 * (size_t)page_size * D * es;
  w.total = off;
  return w;
}

int compact_impl(const int32_t* req_idx, int R, int B, int L, const float* a_short,
                 const float* a_long, int C_max, const int32_t* ws_counts, const int32_t* n_cand,
                 double tau, int k_loc, int policy, const int32_t* policies,
                 gp_kv_cache* const* kv_layers, int32_t* block_tables, int32_t* n_pages,
                 int max_pages, int32_t* context_lens, int32_t* refcount, int32_t* free_stack,
                 int32_t* free_top, int32_t* decision, int32_t* kept_idx, void* workspace,
                 size_t workspace_bytes, int phases, void* stream) {
  if (R < 0 || B < 0 || L <= 0 || C_max <= 0 || !kv_layers || max_pages <= 0 || k_loc < 0)
    return GP_ERR_INVALID;
  if (phases < 1 || phases > (GP_PHASE_PLAN | GP_PHASE_MOVE)) return GP_ERR_INVALID;
  if (R == 0) return GP_OK;
  if (R > DA_MAX_R) return GP_ERR_UNSUPPORTED;
  if (!req_idx || !a_short || !a_long || !ws_counts || !n_cand || !block_tables || !n_pages ||
      !context_lens || !refcount || !free_stack || !free_top || !decision || !kept_idx)
    return GP_ERR_INVALID;
  if (policy < GP_POLICY_AUTO || policy > GP_POLICY_SHRINK) return GP_ERR_INVALID;
  if (!(tau == tau)) return GP_ERR_INVALID;
  const gp_kv_cache* kv = kv_layers[0];
  if (!kv) return GP_ERR_INVALID;
  const int H_kv = kv->num_kv_heads, D = kv->head_dim, b = kv->page_size;
  for (int l = 0; l < L; ++l) {
    const gp_kv_cache* c = kv_layers[l];
    if (!c || !c->k || !c->v) return GP_ERR_INVALID;
    if ((c->page_tag != nullptr) != (kv_layers[0]->page_tag != nullptr)) return GP_ERR_INVALID;
    if (c->num_kv_heads != H_kv || c->head_dim != D || c->page_size != b ||
        c->num_pages != kv->num_pages || c->dtype != kv->dtype)
      return GP_ERR_INVALID;  // the layers share block tables and the page pool
  }
  if (H_kv <= 0 || kv->num_pages <= 0) return GP_ERR_INVALID;
  if (kv->dtype != GP_F32 && kv->dtype != GP_BF16) return GP_ERR_INVALID;
  if (D != 64 && D != 128) return GP_ERR_UNSUPPORTED;
  if (b != 16 && b != 32 && b != 64 && b != 128 && b != 256) return GP_ERR_UNSUPPORTED;
  // a Shrink evicts up to 2b tokens: beyond the 32 evictions of the 32-token path
  if (policy == GP_POLICY_SHRINK && b == 32) return GP_ERR_UNSUPPORTED;
  const bool wide = b >= WIDE_MIN_PAGE;
  // a Shrink moves tokens by up to two pages; only calls where one can occur pay for that
  const int span = (policy == GP_POLICY_SHRINK || policies) ? MAX_SPAN : 1;
  const int es = kv->dtype == GP_F32 ? 4 : 2;
  const int W = wide ? 1 : window_pages_for(b, D, es, span);
  size_t lds;
  if (wide) {
    lds = (size_t)(span + 1) * WIDE_PART * b;
    if (lds + sizeof(int) * (WIDE_MAX_EVICT + 2 * 256) + 16 * (2 * CHUNK_PAGES + MAX_SPAN) > 64 * 1024)
      return GP_ERR_UNSUPPORTED;
  } else {
    lds = (size_t)(W + span) * b * D * es;
    if (lds + sizeof(int) * (MAX_EVICT + MAX_WINDOW_SLOTS) > 64 * 1024) return GP_ERR_UNSUPPORTED;
    if ((long)W * b * D * es > (long)K_PIECES * CP_THREADS * 16) return GP_ERR_UNSUPPORTED;
    if ((long)(W + span) * b * D * es > (long)V_PIECES * CP_THREADS * 16) return GP_ERR_UNSUPPORTED;
  }
  if (C_max % 4 || C_max > MAX_CAND) return GP_ERR_UNSUPPORTED;
  // mixed-precision caches: one layer, bf16 with its fp8 and INT4 pools, 16- or 32-token pages
  const bool mixed = kv->page_tag != nullptr;
  if (mixed) {
    if (L != 1 || kv->dtype != GP_BF16 || wide) return GP_ERR_UNSUPPORTED;
    if (!kv->k8 || !kv->v8 || !kv->k_scale || !kv->v_scale || !kv->k4 || !kv->v4 ||
        !kv->k4_scale || !kv->v4_scale)
      return GP_ERR_INVALID;
  }
  const WsLayout wl = ws_layout(L, R, H_kv, max_pages, b, C_max);
  if (!workspace || workspace_bytes < wl.total) return GP_ERR_WORKSPACE;

  CParams P{};
  P.req_idx = req_idx;
  P.ws_counts = ws_counts;
  P.n_cand = n_cand;
  P.policies = policies;
  P.block_tables = block_tables;
  P.n_pages = n_pages;
  P.context_lens = context_lens;
  P.refcount = refcount;
  P.free_stack = free_stack;
  P.free_top = free_top;
  P.decision = decision;
  P.R = R;
  P.B = B;
  P.L = L;
  P.span = span;
  P.H_kv = H_kv;
  P.D = D;
  P.page_size = b;
  P.num_pages = kv->num_pages;
  P.max_pages = max_pages;
  P.C_max = C_max;
  P.k_loc = k_loc;
  P.policy = policy;
  P.es = es;
  P.tau = tau;
  P.chunk_pages = chunk_pages_for(R, H_kv, b, C_max);
  P.max_chunks = (max_pages + P.chunk_pages - 1) / P.chunk_pages;
  P.window_pages = W;
  P.max_evict = wide ? 2 * b : MAX_EVICT;
  P.npart = wide ? D * es / WIDE_PART : 1;
  P.log_kpq = ilog2(D * es / P.npart / 16);
  // one layer of a uniform cache: the selection lists the compaction items itself
  P.fuse_items = (L == 1 && !mixed) ? 1 : 0;
  P.log_b = ilog2(b);
  P.log_kq = ilog2(D * es / 16);
  P.log_vq = ilog2(b * es / 16);
  P.log_qpp = ilog2(b * D * es / 16);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  P.info = reinterpret_cast<Info*>(ws + wl.info);
  P.old_bt = reinterpret_cast<int32_t*>(ws + wl.old_bt);
  P.rel = reinterpret_cast<int32_t*>(ws + wl.rel);
  P.new_tag = reinterpret_cast<int32_t*>(ws + wl.new_tag);
  P.chk = reinterpret_cast<int32_t*>(ws + wl.chk);
  // many (request, page) pairs: their checks spread over one workgroup per request
  P.split_check = (R >= 2 && (long)R * (C_max / b + 2) > 2 * DA_THREADS) ? 1 : 0;
  if (mixed) {
    P.page_tag = kv->page_tag;
    P.k8 = static_cast<uint8_t*>(kv->k8);
    P.v8 = static_cast<uint8_t*>(kv->v8);
    P.k_scale = kv->k_scale;
    P.v_scale = kv->v_scale;
    P.k4 = static_cast<uint8_t*>(kv->k4);
    P.v4 = static_cast<uint8_t*>(kv->v4);
    P.k4_scale = kv->k4_scale;
    P.v4_scale = kv->v4_scale;
  }
  P.cand = reinterpret_cast<unsigned long long*>(ws + wl.cand);
  P.snap = ws + wl.snap;
  // the parameters of layer l: its scores, kept indices, pools and per-layer workspace
  const size_t plane = (size_t)R * H_kv * C_max;
  auto layer = [&](int l) {
    CParams Q = P;
    Q.a_short = a_short + (size_t)l * plane;
    Q.a_long = a_long + (size_t)l * plane;
    Q.kept_idx = kept_idx + (size_t)l * plane;
    Q.k = static_cast<uint8_t*>(kv_layers[l]->k);
    Q.v = static_cast<uint8_t*>(kv_layers[l]->v);
    uint8_t* lw = ws + wl.layer0 + (size_t)l * wl.layer_bytes;
    Q.ev = reinterpret_cast<int32_t*>(lw + wl.ev);
    Q.dp0 = reinterpret_cast<int32_t*>(lw + wl.dp0);
    Q.items = reinterpret_cast<int4*>(lw + wl.items);
    Q.n_items = reinterpret_cast<int32_t*>(lw + wl.n_items);
    return Q;
  };

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (phases & GP_PHASE_PLAN) {
    // one decision and allocation per request for all layers (Eq. 8 over layers and KV heads)
    if (P.split_check) {
      hipLaunchKernelGGL(page_check_kernel, dim3(R), dim3(PC_THREADS), 0, s, layer(0));
      GP_CHECK_LAUNCH();
    }
    hipLaunchKernelGGL(decide_alloc_kernel, dim3(1), dim3(DA_THREADS), 0, s, layer(0));
    GP_CHECK_LAUNCH();
    const dim3 gw(H_kv, R);
    const int nch = (C_max + SEL_T * b - 1) / (SEL_T * b);  // chunks of the longest candidate set
    for (int l = 0; l < L; ++l) {  // selection per layer and KV head (Eq. 9-10)
      const CParams Q = layer(l);
      if (wide) {
        if (b == 64) hipLaunchKernelGGL(select_wide_kernel<2>, gw, dim3(WIDE_T), 0, s, Q);
        else if (b == 128) hipLaunchKernelGGL(select_wide_kernel<4>, gw, dim3(WIDE_T), 0, s, Q);
        else hipLaunchKernelGGL(select_wide_kernel<8>, gw, dim3(WIDE_T), 0, s, Q);
      } else if (nch <= FUSED_MAX_CHUNKS) {
        if (b == 16) hipLaunchKernelGGL(select_fused_kernel<16>, gw, dim3(SEL_T), 0, s, Q);
        else hipLaunchKernelGGL(select_fused_kernel<32>, gw, dim3(SEL_T), 0, s, Q);
      } else {  // longer candidate sets: the chunks of a head in parallel
        const dim3 g(nch, H_kv, R);
        if (b == 16) hipLaunchKernelGGL(select_local_kernel<16>, g, dim3(SEL_T), 0, s, Q);
        else hipLaunchKernelGGL(select_local_kernel<32>, g, dim3(SEL_T), 0, s, Q);
        GP_CHECK_LAUNCH();
        if (b == 16) hipLaunchKernelGGL(select_write_kernel<16>, g, dim3(SEL_T), 0, s, Q);
        else hipLaunchKernelGGL(select_write_kernel<32>, g, dim3(SEL_T), 0, s, Q);
      }
      GP_CHECK_LAUNCH();
      if (mixed) {  // destination tags; every head rewrites from the first changed page
        hipLaunchKernelGGL(mixed_plan_kernel, dim3((max_pages + PLAN_THREADS - 1) / PLAN_THREADS, R),
                           dim3(PLAN_THREADS), 0, s, Q);
        GP_CHECK_LAUNCH();
      }
      if (!P.fuse_items) {
        hipLaunchKernelGGL(chunk_list_kernel, dim3(1), dim3(DA_THREADS), 0, s, Q);
        GP_CHECK_LAUNCH();
      }
    }
  }
  const int cus = device_cus();
  const int max_items = R * H_kv * P.max_chunks * P.npart;
  // The snapshot only reads K/V pages (into the workspace). With one layer it joins the plan,
  // which may run beside work that reads the same pages; with several layers the layers share
  // the snapshot space, so each layer's snapshot directly precedes its own move.
  auto snapshot = [&](const CParams& Q) {
    if (mixed)
      hipLaunchKernelGGL(snapshot_mixed_kernel, dim3(std::max(1, std::min(4 * cus, max_items))),
                         dim3(CP_THREADS), 0, s, Q);
    else
      hipLaunchKernelGGL(snapshot_kernel, dim3(std::max(1, std::min(4 * cus, max_items))),
                         dim3(CP_THREADS), 0, s, Q);
  };
  if ((phases & GP_PHASE_PLAN) && L == 1) {
    snapshot(layer(0));
    GP_CHECK_LAUNCH();
  }
  if (!(phases & GP_PHASE_MOVE)) return GP_OK;
  for (int l = 0; l < L; ++l) {
    const CParams Q = layer(l);
    if (L > 1) {
      snapshot(Q);
      GP_CHECK_LAUNCH();
    }
    if (mixed) {
      CParams M = Q;
      M.window_pages = mixed_window_pages(b, D, span);
      hipLaunchKernelGGL(compact_mixed_kernel, dim3(std::max(1, std::min(4 * cus, max_items))),
                         dim3(CP_THREADS), (size_t)(M.window_pages + span) * 2 * b * D, s, M);
      GP_CHECK_LAUNCH();
      hipLaunchKernelGGL(mixed_tags_kernel, dim3(R), dim3(256), 0, s, Q);
      GP_CHECK_LAUNCH();
      continue;
    }
    if (wide)  // a multiple of NUM_XCD workgroups (the kernel deals chunks to XCDs)
      hipLaunchKernelGGL(compact_wide_kernel,
                         dim3(NUM_XCD * std::max(1, std::min(4 * cus, max_items) / NUM_XCD)),
                         dim3(CP_THREADS), lds, s, Q);
    else
      hipLaunchKernelGGL(compact_kernel, dim3(std::max(1, std::min(2 * cus, max_items))),
                         dim3(CP_THREADS), lds, s, Q);
    GP_CHECK_LAUNCH();
  }
  return GP_OK;
}

}  // namespace

extern "C" size_t gp_compact_or_grow_layers_workspace_size(int num_layers, int R, int H_kv,
                                                          int max_pages, int page_size,
                                                          int C_max) {
  if (num_layers <= 0 || R <= 0 || H_kv <= 0 || max_pages <= 0 || page_size <= 0) return 0;
  return ws_layout(num_layers, R, H_kv, max_pages, page_size, C_max).total;
}

extern "C" size_t gp_compact_or_grow_workspace_size(int R, int H_kv, int max_pages, int page_size,
                                                   int C_max) {
  return gp_compact_or_grow_layers_workspace_size(1, R, H_kv, max_pages, page_size, C_max);
}

extern "C" int gp_compact_or_grow_layers(const int32_t* req_idx, int R, int B, int num_layers,
                                         const float* a_short, const float* a_long, int C_max,
                                         const int32_t* ws_counts, const int32_t* n_cand,
                                         double tau, int k_loc, int policy,
                                         const int32_t* policies, gp_kv_cache* const* kv_layers,
                                         int32_t* block_tables, int32_t* n_pages, int max_pages,
                                         int32_t* context_lens, int32_t* refcount,
                                         int32_t* free_stack, int32_t* free_top,
                                         int32_t* decision, int32_t* kept_idx, void* workspace,
                                         size_t workspace_bytes, int phases, void* stream) {
  return compact_impl(req_idx, R, B, num_layers, a_short, a_long, C_max, ws_counts, n_cand, tau,
                      k_loc, policy, policies, kv_layers, block_tables, n_pages, max_pages,
                      context_lens, refcount, free_stack, free_top, decision, kept_idx, workspace,
                      workspace_bytes, phases, stream);
}

extern "C" int gp_compact_or_grow_phase(const int32_t* req_idx, int R, int B,
                                        const float* a_short, const float* a_long, int C_max,
                                        const int32_t* ws_counts, const int32_t* n_cand, double tau,
                                        int k_loc, int policy, const int32_t* policies,
                                        gp_kv_cache* kv, int32_t* block_tables, int32_t* n_pages,
                                        int max_pages, int32_t* context_lens, int32_t* refcount,
                                        int32_t* free_stack, int32_t* free_top, int32_t* decision,
                                        int32_t* kept_idx, void* workspace,
                                        size_t workspace_bytes, int phases, void* stream) {
  gp_kv_cache* one[1] = {kv};
  return compact_impl(req_idx, R, B, 1, a_short, a_long, C_max, ws_counts, n_cand, tau, k_loc,
                      policy, policies, kv ? one : nullptr, block_tables, n_pages, max_pages,
                      context_lens, refcount, free_stack, free_top, decision, kept_idx, workspace,
                      workspace_bytes, phases, stream);
}

extern "C" int gp_compact_or_grow(const int32_t* req_idx, int R, int B, const float* a_short,
                                  const float* a_long, int C_max, const int32_t* ws_counts,
                                  const int32_t* n_cand, double tau, int k_loc, int policy,
                                  const int32_t* policies, gp_kv_cache* kv, int32_t* block_tables,
                                  int32_t* n_pages, int max_pages, int32_t* context_lens,
                                  int32_t* refcount, int32_t* free_stack, int32_t* free_top,
                                  int32_t* decision, int32_t* kept_idx, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return gp_compact_or_grow_phase(req_idx, R, B, a_short, a_long, C_max, ws_counts, n_cand, tau,
                                  k_loc, policy, policies, kv, block_tables, n_pages, max_pages,
                                  context_lens, refcount, free_stack, free_top, decision, kept_idx,
                                  workspace, workspace_bytes, GP_PHASE_PLAN | GP_PHASE_MOVE,
                                  stream);
}
