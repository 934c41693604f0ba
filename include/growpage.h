/*
 * growpage.h - C ABI of the MI355X (gfx950) paged-KV decode and page-boundary budgeting library.
 *
 * Operations and the passages that define them:
 *   gp_paged_decode_attn      PASK, Sec. 3.1 (o = V softmax(K^T q / sqrt(d_k))), App. B.2 and B.5
 *                             (mixed-precision pages, GQA routes, split-KV merge); GrowPage Sec. 4.2
 *                             (block tables, unchanged attention interface after a grown page).
 *   gp_quantize_pages_int4    PASK App. B.5 (symmetric per-row INT4 codes with half scales, two
 *                             signed nibbles per byte).
 *   gp_update_query_summaries GrowPage Sec. 3.2 Eq. 6 and App. E.1 (slot pool, first-step init).
 *   gp_score_and_working_set  GrowPage App. E.1 Eq. 12 (RMS calibration + RoPE), Sec. 3.2
 *                             (candidate set without the most recent block, short/long views),
 *                             Eq. 2 / Eq. 7 (p-coverage working set).
 *   gp_compact_or_grow        GrowPage Eq. 8 (trend, tau), Sec. 3.3 Eq. 9-10 (importance and
 *                             block-local + global selection, Compress & Hold, Grow by One Page),
 *                             Sec. 4.2 and App. E.2 (free-page pool, fallback, prefix sharing),
 *                             App. H.1 (fixed / inverse / shrink policies, Eq. 13); the _phase
 *                             and _layers forms split it for overlap (App. E.3) and aggregate
 *                             Eq. 8 over layers.
 *
 * Conventions shared by every call
 *   - All array arguments are DEVICE pointers owned by the caller; scalars are passed by value.
 *     The library allocates no memory: scratch comes from a caller-provided workspace whose size
 *     the matching *_workspace_size() call returns (NULL / 0 allowed when that size is 0).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream) and never
 *     synchronises with the host, so calls can be captured in a HIP graph.
 *   - Return value: GP_OK or a negative gp_status. Arguments are validated on the host before
 *     anything is launched; on error nothing is launched and no buffer is touched.
 *     Values read from device arrays (block-table entries, lengths, slots, request indices)
 *     are range-checked inside the kernels: an entry outside its range makes that request (or
 *     page) count as empty rather than being dereferenced.
 *   - Layouts (row-major, innermost last):
 *       K pool  [num_pages, H_kv, page_size, head_dim]       (a page holds page_size key rows)
 *       V pool  [num_pages, H_kv, head_dim, page_size]       (values transposed within a page)
 *       block_tables [B, max_pages] int32, context_lens [B] int32 (cached tokens of a request;
 *       token slot j lives at page block_tables[r][j / page_size], offset j % page_size).
 *     The query head g uses KV head g / (H_q / H_kv).
 *   - Re-entrant. Calls share no device memory (except gp_paged_decode_attn_noalloc, whose
 *     calls share one static buffer per device) and no host state that affects results. The
 *     only host-side mutable state is three memo tables per device (the compute-unit count, the
 *     resident workgroups of each decode kernel, the device address of the static buffer), each
 *     entry one atomic word, so concurrent calls at worst query the device twice.
 */
#ifndef GROWPAGE_H
#define GROWPAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raised whenever an argument struct or a call's signature changes (2: gp_kv_cache.tags_present). */
#define GP_VERSION 2

typedef enum {
  GP_OK = 0,
  GP_ERR_INVALID = -1,      /* a pointer, size or parameter is out of range            */
  GP_ERR_UNSUPPORTED = -2,  /* a valid combination this build does not implement       */
  GP_ERR_WORKSPACE = -3,    /* workspace missing or smaller than *_workspace_size()     */
  GP_ERR_HIP = -4,          /* a HIP launch failed                                      */
  GP_ERR_SCRATCH = -5       /* the call needs more than GP_NOALLOC_SCRATCH_BYTES        */
} gp_status;

typedef enum { GP_F32 = 0, GP_BF16 = 1 } gp_dtype;

/* Page tags of mixed-precision caches (PASK App. B.2: released entries keep their positions). */
enum { GP_TAG_RELEASE = 0, GP_TAG_FP8 = 1, GP_TAG_BF16 = 2, GP_TAG_INT4 = 3 };

/* Outcome per boundary request (GrowPage Sec. 4.2, App. H.2). */
enum {
  GP_DECISION_COMPRESS = 0,               /* Compress & Hold                                 */
  GP_DECISION_GROW = 1,                   /* Grow by One Page                                */
  GP_DECISION_GROW_FALLBACK_COMPRESS = 2, /* grow wanted, no page granted: compressed instead */
  GP_DECISION_NO_PAGES = 3,               /* neither possible: request left untouched        */
  GP_DECISION_SHRINK = 4                  /* GrowPage-Shrink: two pages' worth evicted, the
                                             last page returned to the pool (App. H.1)       */
};

/* Capacity-control policies (GrowPage Sec. 3.2 and App. H.1). */
enum {
  GP_POLICY_AUTO = 0,           /* grow iff Delta > tau                        */
  GP_POLICY_FORCE_COMPRESS = 1, /* GrowPage-Fixed: always Compress & Hold      */
  GP_POLICY_FORCE_GROW = 2,     /* always try to grow                          */
  GP_POLICY_INVERSE = 3,        /* GrowPage-Inverse: grow iff Delta <= tau     */
  GP_POLICY_SHRINK = 4          /* GrowPage-Shrink (Eq. 13): shrink iff Delta < -0.005, grow iff
                                   Delta > tau, else Compress & Hold                        */
};

/*
 * One layer's paged KV cache.
 *   k, v      pools in `dtype` (GP_F32 or GP_BF16), layouts above. Required.
 *   page_tag  NULL for a uniform cache. Otherwise [num_pages] uint8 with GP_TAG_*: a mixed
 *             cache (dtype must be GP_BF16) whose fp8 and INT4 pools must all be given.
 *             Released pages are skipped entirely; bf16 pages read k/v; fp8 pages read k8/v8
 *             (OCP E4M3FN codes, same layouts as k/v) times the per-row scales
 *             k_scale/v_scale [num_pages, H_kv, page_size] fp32; INT4 pages (PASK App. B.5)
 *             read signed 4-bit codes (two's complement nibbles, the even index of a pair in
 *             the low nibble) times per-row IEEE half scales:
 *               k4       [num_pages, H_kv, page_size, head_dim / 2]  key rows packed along d
 *               v4       [num_pages, H_kv, page_size / 4, head_dim, 2]  values packed along
 *                        the token axis in blocks of 4 tokens: byte 0 of a dimension holds
 *                        tokens 4Q, 4Q+1, byte 1 tokens 4Q+2, 4Q+3; within a block dimension
 *                        j sits at position (j % 16) * (head_dim / 16) + j / 16, so that the
 *                        head_dim / 16 dimensions one lane accumulates are adjacent
 *               k4_scale, v4_scale [num_pages, H_kv, page_size]      half bits, one per token
 *                        row and KV head.
 *             A byte value in an INT4 pool always decodes to finite codes (-8 .. 7), so only
 *             the scales of live tokens need to be meaningful.
 *             A uniformly fp8 cache is a mixed cache whose pages are all tagged GP_TAG_FP8 (the
 *             bf16 and INT4 pools are then never read, but must still be given).
 *   page_size a multiple of 16 (16 .. 256); head_dim 64 or 128.
 *   tags_present  mixed caches only, read by the decode calls: 0 (unknown: every pass runs), or
 *             the set of page tags (bit 1 << GP_TAG_*) that the pages the block tables reach may
 *             carry. A mixed decode runs one pass over the bf16 and fp8 pages and one over the
 *             INT4 pages; a pass whose tags are all absent from the set is not launched (with no
 *             bf16, fp8 or INT4 bit at all, the first pass still runs). A launched pass decodes
 *             every page of its tags, declared or not; the pages of a pass that is not launched
 *             are skipped exactly like released pages. The set is a promise of the caller:
 *             breaking it loses those pages' tokens, nothing more (no read outside the pools).
 *             The score and compaction calls read every page's tag and ignore this field.
 */
typedef struct {
  void* k;
  void* v;
  void* k8;
  void* v8;
  float* k_scale;
  float* v_scale;
  uint8_t* page_tag; /* written by gp_quantize_pages_int4 and by mixed-cache compaction */
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;
  void* k4;
  void* v4;
  uint16_t* k4_scale;
  uint16_t* v4_scale;
  uint32_t tags_present;
} gp_kv_cache;

int gp_version(void);
const char* gp_status_string(int status);

/*
 * Decode attention for one new token per request (PASK Sec. 3.1, App. B.5).
 *   q            [B, H_q, head_dim] in the cache dtype (bf16 for mixed caches); the query as
 *                attention sees it (already rotated).
 *   block_tables [B, max_pages]; context_lens [B] (0 .. max_context; 0 gives out = 0, lse = -inf).
 *   max_context  host-side upper bound on every context_lens[r]; it sizes the workspace.
 *   sm_scale     logit scale, normally 1/sqrt(head_dim).
 *   out          [B, H_q, head_dim] in the q dtype.
 *   lse          [B, H_q] fp32 natural-log log-sum-exp of the scaled logits, or NULL.
 *   workspace    >= gp_paged_decode_attn_workspace_size(...) bytes: a prefix of the per-request
 *                tile counts and the partial (max, sum, output) of every request segment. Its
 *                contents need no initialisation and are meaningless after the call.
 * The 16-token tiles of the whole batch are divided evenly over the resident workgroups; a
 * request spread over several of them is merged from its partials with PASK App. B.5's rule.
 * Limits: B <= 8191, 1 <= H_q / H_kv <= 16, head_dim 64 or 128, page_size a multiple of 16 up to
 * 256. Any H_kv (a workgroup takes the largest divisor of H_kv up to 8 KV heads).
 * INT4 pages are contracted exactly in half precision: the query elements are rounded to half
 * (exact for bf16 values of magnitude 2^-14 .. 65504; larger ones overflow) and the probability
 * weights times the value scales are rounded to half toward zero before the value product.
 */
size_t gp_paged_decode_attn_workspace_size(int B, int H_q, int H_kv, int head_dim, int page_size,
                                           int max_context);
int gp_paged_decode_attn(const void* q, int q_dtype, int B, int H_q, const gp_kv_cache* kv,
                         const int32_t* block_tables, int max_pages, const int32_t* context_lens,
                         int max_context, float sm_scale, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Demote bf16 pages of a mixed cache to INT4 pages (PASK App. B.5).
 *   page_ids [num_ids] int32 device array. For every listed page whose tag is GP_TAG_BF16, each
 *   K row and each V row (one token of one KV head, head_dim elements read from k / v) gets the
 *   scale s = half(amax / 7) (nearest, ties to even; at least 2^-24; 1 for an all-zero row)
 *   written to k4_scale / v4_scale, and the codes clip(round_half_even(x / s), -7, 7) written
 *   to k4 / v4 in the layouts of gp_kv_cache; then the tag becomes GP_TAG_INT4. All page_size
 *   rows of the page are converted. Ids outside [0, num_pages) and pages with another tag are
 *   left alone; a repeated id is converted once. The bf16 pool of the page is not modified.
 *   Rows holding NaN or Inf get unspecified codes and scales.
 *   kv must be a mixed cache (page_tag, k4, v4, k4_scale, v4_scale given, dtype GP_BF16).
 */
int gp_quantize_pages_int4(const gp_kv_cache* kv, const int32_t* page_ids, int num_ids,
                           void* stream);

/*
 * Decode attention with the summary update fused in (GrowPage Sec. 4.1: the attention kernel also
 * updates both EMA summaries from the pre-RoPE query), and an optional cap on its grid.
 *   Arguments as gp_paged_decode_attn (same workspace size), plus
 *   summaries       NULL, or the update of gp_update_query_summaries applied to every request
 *                   of this call (the same arithmetic, so the same bits); it is finished when
 *                   the call's work on the stream is.
 *   max_workgroups  0, or an upper bound on the workgroups of the streaming kernel (at least one
 *                   per group of 8 KV heads is kept), so that kernels on another stream find
 *                   free compute units while this call runs. With a cap, a bf16 or fp32 cache is
 *                   decoded with one tile in flight per wave instead of two (shorter memory
 *                   queues for the kernels beside it); results are the same bits either way.
 */
typedef struct {
  const void* q_pre;       /* [B, H_q, head_dim] pre-RoPE queries, in q_dtype                 */
  const int32_t* slot_ids; /* [B] slot of each request in [0, num_slots); others are skipped  */
  const uint8_t* fresh;    /* [B] 1 = first step of the slot: both summaries = q_pre          */
  float* qstate;           /* [num_slots, 2, H_q, head_dim] fp32, updated in place            */
  int num_slots;
  float beta_s, beta_l;
} gp_summary_update;

int gp_paged_decode_attn_ex(const void* q, int q_dtype, int B, int H_q, const gp_kv_cache* kv,
                            const int32_t* block_tables, int max_pages,
                            const int32_t* context_lens, int max_context, float sm_scale,
                            void* out, float* lse, const gp_summary_update* summaries,
                            int max_workgroups, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * gp_paged_decode_attn_ex without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * split partials live in a static device buffer of GP_NOALLOC_SCRATCH_BYTES that the library
 * holds on every device it runs on until the process ends. Arguments, results and bits as
 * gp_paged_decode_attn_ex. The call allocates nothing (no hipMalloc, no library allocation).
 *   Limit: the call needs the prefix of tile counts plus B * H_q * passes * j_max * (head_dim + 2)
 *   floats of partials (passes = 2 for a mixed cache, else 1; j_max grows with max_context and
 *   shrinks with B, as gp_paged_decode_attn_workspace_size counts them); a call needing more
 *   than GP_NOALLOC_SCRATCH_BYTES returns GP_ERR_SCRATCH and launches nothing.
 *   Every call on one device shares that device's buffer: calls that may overlap on one device
 *   (other streams, other threads) race and must be ordered by the caller. Nothing in the
 *   buffer needs clearing between calls (each call writes what it reads).
 */
#define GP_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gp_paged_decode_attn_noalloc(const void* q, int q_dtype, int B, int H_q,
                                 const gp_kv_cache* kv, const int32_t* block_tables,
                                 int max_pages, const int32_t* context_lens, int max_context,
                                 float sm_scale, void* out, float* lse,
                                 const gp_summary_update* summaries, int max_workgroups,
                                 void* stream);

/*
 * Dual-timescale EMA of the pre-RoPE queries (GrowPage Eq. 6, App. E.1).
 *   q        [B, H_q, head_dim] (GP_F32 or GP_BF16).
 *   slot_ids [B] int32 in [0, num_slots); fresh [B] uint8 (1 = first step of this slot).
 *   qstate   [num_slots, 2, H_q, head_dim] fp32, index 0 short and 1 long; updated in place:
 *            fresh: both = q; else x <- beta_x * x + (1 - beta_x) * q.
 * Two requests of one call must not share a slot.
 */
int gp_update_query_summaries(const void* q, int q_dtype, int B, int H_q, int head_dim,
                              const int32_t* slot_ids, const uint8_t* fresh, float* qstate,
                              int num_slots, float beta_s, float beta_l, void* stream);

/*
 * Scores and working sets of the boundary requests (GrowPage App. E.1, Sec. 3.2, Eq. 7, Eq. 12).
 *   q [B, H_q, head_dim] current pre-RoPE queries; qstate / slot_ids as above.
 *   req_idx [R] request indices in [0, B); positions [B] 0-based position of the current token.
 *   For request r the candidate set C is every slot outside its last (partially) filled page:
 *   |C| = (ceil(ctx/b) - 1) * b. Per query head and view x in {short, long} the summary is
 *   RMS-calibrated to q (Eq. 12), rotated (rotate-half RoPE on pairs (i, i + d/2), angle
 *   pos * rope_theta^(-2i/d); rope_theta <= 0 disables it), and softmax-ed over C with scale
 *   sm_scale; the G query heads of a KV head are averaged.
 *   a_short, a_long [R, H_kv, C_max] fp32 outputs; entries past |C| are not written.
 *   ws_counts [R, H_kv, 2] int32: K^S, K^L = min{k : sum of the k largest weights >= p},
 *   computed exactly on the fp32 weights written to a_short / a_long (|C| if never reached).
 *   n_cand [R] int32 = |C|; a request whose index, slot or length is out of range, or whose
 *   |C| exceeds C_max, gets n_cand = -1 and ws_counts = -1 and is otherwise skipped.
 *   Limits: 2 * (H_q / H_kv) <= 16, C_max <= 32768 and a multiple of 4, 0 < p <= 1.
 *   workspace >= gp_score_and_working_set_workspace_size(...) bytes.
 *   Mixed-precision caches (page_tag given; GP_BF16 with the fp8 and INT4 key pools): an fp8
 *   key is its E4M3 code value times the row scale, an INT4 key its signed nibbles times the
 *   row's half scale (PASK App. B.5), and the tokens of released pages take no part in the
 *   softmax (weight 0; |C| still counts their slots).
 */
size_t gp_score_and_working_set_workspace_size(int R, int H_q, int H_kv, int head_dim,
                                               int page_size, int C_max);
int gp_score_and_working_set(const void* q, int q_dtype, int B, int H_q, const float* qstate,
                             int num_slots, const int32_t* slot_ids, const int32_t* req_idx, int R,
                             const gp_kv_cache* kv, const int32_t* block_tables, int max_pages,
                             const int32_t* context_lens, const int32_t* positions,
                             float rope_theta, double p, float sm_scale, float* a_short,
                             float* a_long, int C_max, int32_t* ws_counts, int32_t* n_cand,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Compress-or-grow for the boundary requests, processed in req_idx order (GrowPage Sec. 3.2,
 * Sec. 3.3, Sec. 4.2, App. E.2, App. H.1).
 *   Decision: Delta = (1/H_kv) sum_h (K^S_h - K^L_h) / |C| compared exactly with tau under
 *   `policy` (or policies[i] when `policies` is non-NULL); |C| = 0 always grows. Under
 *   GP_POLICY_SHRINK a request with Delta < -0.005 (exact) shrinks instead of compressing when
 *   its capacity stays >= 1024 tokens afterwards ((n_pages - 1) * page_size >= 1024): as
 *   Compress below with K_t = min(|C|, (P-2)b - |R|), then the last page leaves the block table
 *   (n_pages - 1) and its reference is released after the request's replaced pages.
 *   Grow: pop free_stack[*free_top - 1], append it to the block table, n_pages += 1, refcount
 *   of the page = 1. No free page (or a full block table) falls back to compression.
 *   Compress: with P = n_pages[r], R = tokens of the last page, K_t = min(|C|, (P-1)b - |R|).
 *   If K_t < |C|, each page among the first ceil((K_t+|R|)/b) that is shared (refcount > 1)
 *   is replaced by a popped page (ascending logical order; too few free pages -> NO_PAGES,
 *   request untouched), then per KV head the kept set S (Eq. 9-10 with k_loc, ties to the lower
 *   token index) in ascending order followed by the |R| recent tokens is written to slots
 *   0 .. K_t+|R|-1 and context_lens[r] becomes K_t + |R|. Released references are
 *   decremented after all pops of the call; pages reaching zero are pushed on the stack.
 *   decision [R] int32 (GP_DECISION_*); kept_idx [R, H_kv, C_max] int32: within the first |C|
 *   entries of a row, the kept candidate indices in ascending order (all of C when nothing is
 *   evicted) and -1 after them, or -1 throughout for requests that grew or got no pages;
 *   entries past |C| are not written.
 *   a_short / a_long / ws_counts / n_cand as produced by gp_score_and_working_set.
 *   kv, block_tables, n_pages, context_lens, refcount, free_stack, free_top are updated in place.
 *   Requests of one call must be distinct.
 *   workspace: at least gp_compact_or_grow_workspace_size(R, H_kv, max_pages, page_size, C_max)
 *   bytes for this call's R and C_max (the size, like the length of the compaction's work items,
 *   depends on them), otherwise GP_ERR_WORKSPACE.
 *   Mixed-precision caches (page_tag given; GP_BF16 with every fp8 and INT4 pool; pages of 16
 *   or 32 tokens; one layer): a request that must move tokens while one of its pages is
 *   released is answered NO_PAGES and left untouched (one tag per page cannot keep a released
 *   token masked among live ones). Otherwise every KV head rewrites the pages from the first
 *   one that changes for any head; a destination page keeps a precision when all the pages
 *   that supply its tokens (any head) carry it, and the tokens move with their codes and row
 *   scales bit for bit (INT4 value nibbles regrouped into four-token blocks); else it becomes a
 *   bf16 page holding each token's code * scale rounded once to bf16 (nearest, ties to even).
 *   page_tag of the rewritten pages is updated at the end of the move.
 *   Limits: R <= 1024, page_size 16, 32, 64, 128 or 256 (32-token fp32 pages need head_dim
 *   64), C_max <= 32768 and a multiple of 4. A Shrink evicts up to 2 * page_size tokens: with
 *   32-token pages GP_POLICY_SHRINK is rejected and a per-request Shrink is answered NO_PAGES.
 *   With pages of 64 tokens or more (GrowPage's own runs use 256-token blocks and k_loc = 64)
 *   the candidate set still excludes the whole last page, so all of its tokens are kept.
 */
size_t gp_compact_or_grow_workspace_size(int R, int H_kv, int max_pages, int page_size, int C_max);

/*
 * gp_compact_or_grow in two phases, so that the data movement can be scheduled apart from the
 * bookkeeping (GrowPage App. E.3 overlaps compaction with decoding):
 *   GP_PHASE_PLAN  decisions, page allocation and release, kept_idx, and the list of page chunks
 *                  to move: every update of block_tables, n_pages, context_lens, refcount,
 *                  free_stack, free_top and decision. K/V pages are not written (with one
 *                  layer the plan also copies the few pages the move will need into the
 *                  workspace: reads only).
 *   GP_PHASE_MOVE  the K/V movement planned by the PLAN call that used this workspace; it must
 *                  come after that call (same arguments and workspace, none of them changed in
 *                  between) and after every read of the boundary requests' old pages.
 * phases = GP_PHASE_PLAN | GP_PHASE_MOVE is gp_compact_or_grow itself.
 */
enum { GP_PHASE_PLAN = 1, GP_PHASE_MOVE = 2 };

/*
 * Compress-or-grow for L layers that share block tables and the page pool (GrowPage Eq. 8:
 * one decision per request from the mean of (K^S - K^L)/|C| over every layer and KV head;
 * Eq. 9-10: selection and compaction per layer and KV head).
 *   a_short, a_long, kept_idx  [num_layers, R, H_kv, C_max] (layer l's scores at offset l);
 *   ws_counts                  [num_layers, R, H_kv, 2];
 *   kv_layers                  HOST array of num_layers caches with the same geometry and dtype;
 *   n_cand [R] (the candidate count does not depend on the layer); other arguments, phases and
 *   outcomes as gp_compact_or_grow_phase. num_layers = 1 is gp_compact_or_grow_phase itself.
 *   workspace >= gp_compact_or_grow_layers_workspace_size(num_layers, ...) bytes.
 */
size_t gp_compact_or_grow_layers_workspace_size(int num_layers, int R, int H_kv, int max_pages,
                                                int page_size, int C_max);
int gp_compact_or_grow_layers(const int32_t* req_idx, int R, int B, int num_layers,
                              const float* a_short, const float* a_long, int C_max,
                              const int32_t* ws_counts, const int32_t* n_cand, double tau,
                              int k_loc, int policy, const int32_t* policies,
                              gp_kv_cache* const* kv_layers, int32_t* block_tables,
                              int32_t* n_pages, int max_pages, int32_t* context_lens,
                              int32_t* refcount, int32_t* free_stack, int32_t* free_top,
                              int32_t* decision, int32_t* kept_idx, void* workspace,
                              size_t workspace_bytes, int phases, void* stream);
int gp_compact_or_grow_phase(const int32_t* req_idx, int R, int B, const float* a_short,
                             const float* a_long, int C_max, const int32_t* ws_counts,
                             const int32_t* n_cand, double tau, int k_loc, int policy,
                             const int32_t* policies, gp_kv_cache* kv, int32_t* block_tables,
                             int32_t* n_pages, int max_pages, int32_t* context_lens,
                             int32_t* refcount, int32_t* free_stack, int32_t* free_top,
                             int32_t* decision, int32_t* kept_idx, void* workspace,
                             size_t workspace_bytes, int phases, void* stream);
int gp_compact_or_grow(const int32_t* req_idx, int R, int B, const float* a_short,
                       const float* a_long, int C_max, const int32_t* ws_counts,
                       const int32_t* n_cand, double tau, int k_loc, int policy,
                       const int32_t* policies, gp_kv_cache* kv, int32_t* block_tables,
                       int32_t* n_pages, int max_pages, int32_t* context_lens, int32_t* refcount,
                       int32_t* free_stack, int32_t* free_top, int32_t* decision,
                       int32_t* kept_idx, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GROWPAGE_H */
