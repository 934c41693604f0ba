"""GrowPage's page-boundary pass, float64 / exact integer arithmetic.

Steps, in the order GrowPage App. E.1 runs them at a capacity boundary:

1. Calibration (Eq. 12): gamma^x = RMS(q_t) / RMS(qbar^x), qtilde^x = gamma^x qbar^x, then RoPE
   at the current decoding position (Sec. 3.2, App. E.1). RoPE here is the rotate-half form
   on pairs (i, i + d/2) with angle pos * theta^(-2i/d); theta <= 0 disables it.
2. Candidate set C_t: every cached slot outside the most recent page (Sec. 3.2, App. E.1
   "exclude the most recent physical KV block"). The slots of that last page are the
   protected recent tokens R_t of Sec. 3.3. With pages longer than the 16-token recent
   window of Sec. 4.1 (its runs use 256-token blocks) the window lies inside that page, and
   Eq. 10 selects only from C_t, so every token of the last page is kept.
3. Scores: for each view x and KV head h, the softmax over C_t of qtilde^x_g . k / sqrt(d) for
   each query head g mapped to h (native GQA mapping, App. E.1), averaged over those heads.
4. Working set (Eq. 2 / Eq. 7): K^x_h = min{k : sum of the k largest weights >= p}, computed
   exactly on the given weight values; if no k reaches p, K = |C_t|.
5. Trend and decision (Eq. 8, Sec. 3.2): Delta = (1/(L H)) sum over layers and KV heads of
   (K^S - K^L) / |C_t| (one decision per request for all layers); Grow by One Page iff
   Delta > tau, else Compress & Hold. Policies of App. H.1: always compress (GrowPage-Fixed),
   always grow, GrowPage-Inverse (grow iff Delta <= tau) and GrowPage-Shrink (Eq. 13): Shrink
   iff Delta < -0.005, grow iff Delta > tau, else Compress & Hold. Shrink evicts two pages'
   worth of history, returns the last page to the pool and leaves one page of free slots; it
   is taken only while the capacity stays at least 1024 tokens afterwards (else Compress &
   Hold).
6. Allocation (Sec. 4.2, App. E.2): Grow pops the top of the global free-page stack and appends
   it to the block table; with no free page (or a full block table) it falls back to
   compression. Compression that must write into pages shared with other requests
   (refcount > 1) first pops one private target page per shared page, in ascending logical
   order; the old references are released after every pop of the call, and a page whose
   count reaches zero is pushed back on the stack. If too few pages are free, the request is
   left untouched (NO_PAGES).
7. Selection (Eq. 9, Eq. 10): s_i = max(a^S_i, a^L_i); K_t = (P - 1) b - |R_t|; S_loc is the
   union over historical pages of their k_loc best tokens; the rest of the budget is filled
   with the best tokens of C_t outside S_loc. Order: larger s first, lower token index first
   on ties. If |S_loc| >= K_t, S is the K_t best tokens of C_t.
8. Compaction (Sec. 3.3, App. E.2): the kept tokens in ascending order, then R_t, are written to
   slots 0 .. K_t + |R_t| - 1 of the (new) block table; the cached length becomes K_t + |R_t|,
   i.e. (P - 1) b, leaving one page of free slots. Selection and compaction run per layer and
   KV head on the shared block table. Shrink uses K_t = (P - 2) b - |R_t|, then drops the last
   page from the block table and releases it with the other references of the call.

Pinned by: RMS of the calibrated summary equals RMS(q_t); RoPE keeps norms and its dot
products depend only on relative position; full retention (p -> 1) gives K = |C|; uniform
weights give K = ceil(p |C|); one dominant weight gives K = 1; brute force over all subsets of
tiny candidate sets (GrowPage Thm. 3.1 / App. C: the top-k weights maximise retained mass);
the tight worst-case construction of App. C; equal summaries give Delta = 0 -> compress and
the inverse policy flips it; selection against brute-force enumeration, and in closed form for
256-token pages with a 64-token quota under monotone scores; page conservation,
refcount bookkeeping, shared pages untouched and kept K/V bit-identical after compaction;
hand-worked GrowPage-Shrink decisions over several layers (tests/golden/shrink_cases.txt); a
shrink's geometry, capacity floor, released page and moved K/V; a call over two layers whose
mean decides, with each layer's moved K/V bit-identical to its own kept set, and one layer
through the layered call equal to the single-layer call.
"""
from fractions import Fraction

import numpy as np

from .fp8 import e4m3_decode
from .int4 import pack_pairs, pack_values, unpack_pairs, unpack_values

TAG_RELEASE, TAG_FP8, TAG_BF16, TAG_INT4 = 0, 1, 2, 3

COMPRESS, GROW, GROW_FALLBACK_COMPRESS, NO_PAGES, SHRINK = 0, 1, 2, 3, 4
POLICY_AUTO, POLICY_FORCE_COMPRESS, POLICY_FORCE_GROW, POLICY_INVERSE, POLICY_SHRINK = 0, 1, 2, 3, 4
SHRINK_BELOW = Fraction(-5, 1000)   # GrowPage Eq. 13
MIN_CAPACITY = 1024                 # tokens a shrink must leave (GrowPage App. H.1)


# ---------------------------------------------------------------------------- step 1
def rms(x):
    x = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.mean(x * x, axis=-1))


def calibrate(q_t, qbar):
    """Eq. 12 for one head: scale qbar so its RMS equals RMS(q_t). A zero summary stays zero."""
    rq, rb = rms(q_t), rms(qbar)
    if rb == 0.0:
        return np.zeros_like(np.asarray(qbar, dtype=np.float64))
    return (rq / rb) * np.asarray(qbar, dtype=np.float64)


def rope(x, pos, theta):
    """Rotate-half RoPE of vectors x [..., d] at integer position pos (theta <= 0: identity)."""
    x = np.asarray(x, dtype=np.float64)
    if theta <= 0:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


# ---------------------------------------------------------------------------- step 2
def candidate_count(ctx, page_size):
    """|C_t|: slots outside the last (partially) filled page."""
    ctx = int(ctx)
    if ctx <= 0:
        return 0
    used = -(-ctx // page_size)
    return (used - 1) * page_size


# ---------------------------------------------------------------------------- step 3
def score_request(q_t, qbar, pos, keys, theta, sm_scale, G, visible=None):
    """Averaged short/long attention over the candidate keys.

    q_t [H_q, d], qbar [2, H_q, d], keys [H_kv, n_cand, d] -> a [2, H_kv, n_cand]. Candidates
    with visible = False (tokens of released pages) take no part in the softmax: weight 0.
    """
    H_kv, n, _ = keys.shape
    a = np.zeros((2, H_kv, n))
    vis = np.ones(n, dtype=bool) if visible is None else np.asarray(visible, dtype=bool)
    if n == 0 or not vis.any():
        return a
    for x in range(2):
        for h in range(H_kv):
            acc = np.zeros(n)
            for g in range(h * G, (h + 1) * G):
                qt = rope(calibrate(q_t[g], qbar[x, g]), pos, theta)
                z = keys[h][vis] @ qt * sm_scale
                w = np.exp(z - z.max())
                acc[vis] += w / w.sum()
            a[x, h] = acc / G
    return a


def candidate_keys(r, n, k_pool, block_tables, page_size, mixed=None):
    """Keys of request r's first n slots as float64 [H_kv, n, d] and their visibility.

    With mixed-precision pages (`mixed`: page_tag, k8, k_scale, k4, k4_scale) an fp8 key is its
    E4M3 code value times the row scale, an INT4 key its signed nibbles times the row's half
    scale (PASK App. B.5), and the tokens of released pages are not visible.
    """
    b = page_size
    slots = np.arange(n)
    pages = np.asarray(block_tables[r])[slots // b].astype(np.int64)
    offs = slots % b
    keys = np.asarray(k_pool)[pages, :, offs, :].astype(np.float64)          # [n, H, d]
    vis = np.ones(n, dtype=bool)
    if mixed is not None and n:
        tags = np.asarray(mixed["page_tag"])[pages]
        vis = tags != TAG_RELEASE
        f8 = tags == TAG_FP8
        if f8.any():
            kc = e4m3_decode(np.asarray(mixed["k8"])[pages[f8], :, offs[f8], :])
            ks = np.asarray(mixed["k_scale"])[pages[f8], :, offs[f8]].astype(np.float64)
            keys[f8] = kc * ks[..., None]
        i4 = tags == TAG_INT4
        if i4.any():
            kc = unpack_pairs(np.asarray(mixed["k4"])[pages[i4], :, offs[i4], :], axis=-1)
            ks = np.asarray(mixed["k4_scale"])[pages[i4], :, offs[i4]].astype(np.float64)
            keys[i4] = kc.astype(np.float64) * ks[..., None]
        keys[~vis] = 0.0
    return keys.transpose(1, 0, 2), vis


# ---------------------------------------------------------------------------- step 4
def _exact_ints(values):
    """Exact integer numerators of float values over a common power-of-two denominator."""
    vals = np.asarray(values)
    scale_exp = 149 if vals.dtype == np.float32 else 1074
    out = []
    for v in vals.tolist():
        num, den = float(v).as_integer_ratio()
        out.append(num * ((1 << scale_exp) // den))
    return out, scale_exp


def working_set_size(weights, p):
    """Eq. 2 / Eq. 7 on the exact values of `weights` (float32 or float64 array)."""
    w = np.asarray(weights)
    n = w.shape[0]
    if n == 0:
        return 0
    desc = np.sort(w)[::-1]
    ints, e = _exact_ints(desc)
    pf = Fraction(p)
    target_num, target_den = pf.numerator << e, pf.denominator   # p * 2^e as a fraction
    total = 0
    for k, v in enumerate(ints, 1):
        total += v
        if total * target_den >= target_num:
            return k
    return n


def score_and_working_set(q, qstate, slot_ids, req_idx, k_pool, block_tables, context_lens,
                          positions, page_size, rope_theta, p, sm_scale, C_max=None, mixed=None):
    """Steps 1-4 for the boundary requests req_idx (`mixed`: see candidate_keys).

    Returns a_short, a_long [R, H_kv, C_max] (float64, zero beyond |C|), ws_counts
    [R, H_kv, 2] (K^S, K^L computed on the float64 weights) and n_cand [R].
    """
    q = np.asarray(q, dtype=np.float64)
    kp = np.asarray(k_pool)
    H_kv = kp.shape[1]
    H_q = q.shape[1]
    G = H_q // H_kv
    R = len(req_idx)
    ncs = [candidate_count(context_lens[r], page_size) for r in req_idx]
    if C_max is None:
        C_max = max(ncs) if ncs else 0
    a_s = np.zeros((R, H_kv, C_max))
    a_l = np.zeros((R, H_kv, C_max))
    ws = np.zeros((R, H_kv, 2), dtype=np.int64)
    for i, r in enumerate(req_idx):
        n = ncs[i]
        keys, vis = candidate_keys(r, n, kp, block_tables, page_size, mixed)
        a = score_request(q[r], np.asarray(qstate[int(slot_ids[r])], dtype=np.float64),
                          int(positions[r]), keys, rope_theta, sm_scale, G, vis)
        a_s[i, :, :n] = a[0]
        a_l[i, :, :n] = a[1]
        for h in range(H_kv):
            ws[i, h, 0] = working_set_size(a[0, h], p)
            ws[i, h, 1] = working_set_size(a[1, h], p)
    return a_s, a_l, ws, np.array(ncs, dtype=np.int64)


def working_set_counts(a_short, a_long, n_cand, p):
    """Step 4 alone, on given weight arrays (the GPU's float32 scores in parity tests)."""
    R, H, _ = a_short.shape
    ws = np.zeros((R, H, 2), dtype=np.int64)
    for i in range(R):
        n = int(n_cand[i])
        for h in range(H):
            ws[i, h, 0] = working_set_size(a_short[i, h, :n], p)
            ws[i, h, 1] = working_set_size(a_long[i, h, :n], p)
    return ws


# ---------------------------------------------------------------------------- step 5
def trend(ws_counts_r, n_cand_r):
    """Eq. 8 as an exact fraction: the mean over every (layer, KV head) row of
    (K^S - K^L) / |C|. ws_counts_r holds rows of (K^S, K^L), layers and heads in any order."""
    ws = np.asarray(ws_counts_r, dtype=np.int64).reshape(-1, 2)
    return Fraction(int(ws[:, 0].sum() - ws[:, 1].sum()), ws.shape[0] * int(n_cand_r))


def primary_action(ws_counts_r, n_cand_r, tau, policy):
    """Primary decision of one request before allocation: "grow", "compress" or "shrink"."""
    if policy == POLICY_FORCE_COMPRESS:
        return "compress"
    if policy == POLICY_FORCE_GROW or n_cand_r == 0:
        return "grow"
    delta = trend(ws_counts_r, n_cand_r)
    grow = delta > Fraction(tau)
    if policy == POLICY_INVERSE:
        grow = not grow
    if grow:
        return "grow"
    if policy == POLICY_SHRINK and delta < SHRINK_BELOW:
        return "shrink"
    return "compress"


def wants_grow(ws_counts_r, n_cand_r, tau, policy):
    """Primary decision of one request (before allocation): True = Grow by One Page."""
    return primary_action(ws_counts_r, n_cand_r, tau, policy) == "grow"


# ---------------------------------------------------------------------------- step 7
def select_kept(s, K_t, page_size, k_loc):
    """Eq. 10 for one (layer, KV head): sorted indices of the K_t retained candidates."""
    s = np.asarray(s, dtype=np.float64)
    n = s.shape[0]
    if K_t >= n:
        return np.arange(n)
    idx = np.arange(n)
    local = []
    for j in range(0, n, page_size):
        blk = idx[j:j + page_size]
        order = blk[np.lexsort((blk, -s[blk]))]
        local.extend(order[:k_loc].tolist())
    local = np.array(sorted(local), dtype=np.int64)
    glob = idx[np.lexsort((idx, -s))]
    if len(local) >= K_t:
        chosen = glob[:K_t]
    else:
        mask = np.ones(n, dtype=bool)
        mask[local] = False
        rest = glob[mask[glob]][:K_t - len(local)]
        chosen = np.concatenate([local, rest])
    return np.sort(chosen)


# ---------------------------------------------------------------------------- mixed pages
def bf16_bits(x):
    """bfloat16 bit patterns (uint16) of float64 values rounded to nearest, ties to even: 8
    significant bits, the subnormal spacing 2^-133 below 2^-126."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                           # |x| = m 2^e with 0.5 <= m < 1
    ulp = np.maximum(e - 8, -133)
    y = np.ldexp(np.rint(np.ldexp(x, -ulp)), ulp)   # exact scalings around one rounding
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _move_mixed(kp, vp, mx, old_bt, new_bt, srcs, first_repl, ctx_new, b, P):
    """Compaction of one layer of a mixed-precision cache for one request.

    srcs[h][j] is the source slot of destination slot j of KV head h. Pages from the first one
    that changes for any head (an evicted token or a replaced page) to the last destination
    page are rewritten for every head. A destination page keeps a precision when every page
    that supplies it a token (any head) has that tag, and the tokens move with their codes and
    row scales bit for bit; otherwise it becomes a bf16 page and each token it receives is
    stored as its dequantised value rounded to bf16 once. kp / vp are the bf16 pools as 16-bit
    patterns; the pools in `mx` and its page_tag are updated in place.
    """
    n_dest = ctx_new // b
    dpm = first_repl
    for src in srcs:
        moved = np.nonzero(src[:ctx_new] != np.arange(ctx_new))[0]
        if len(moved):
            dpm = min(dpm, int(moved[0]) // b)
    tags = mx["page_tag"]
    old_tag = np.asarray(tags)[old_bt[:P]].copy()
    new_tag = {}
    for dp in range(dpm, n_dest):
        # the old pages that supply at least one token of this page, in any head
        supply = {int(sl) // b for src in srcs for sl in src[dp * b:(dp + 1) * b]}
        ts = {int(old_tag[pg]) for pg in supply}
        new_tag[dp] = ts.pop() if len(ts) == 1 else TAG_BF16
    kb, vb = kp.view(np.uint16), vp.view(np.uint16)
    old = {name: np.asarray(mx[name]).copy() for name in
           ("k8", "v8", "k_scale", "v_scale", "k4", "v4", "k4_scale", "v4_scale")}
    kb0, vb0 = kb.copy(), vb.copy()
    vwork = {}
    for h, src in enumerate(srcs):
        for j in range(dpm * b, ctx_new):
            sl = int(src[j])
            sp, so, ts = int(old_bt[sl // b]), sl % b, int(old_tag[sl // b])
            dp, do = j // b, j % b
            pd, td = int(new_bt[dp]), new_tag[dp]
            if td == ts == TAG_BF16:
                kb[pd, h, do, :] = kb0[sp, h, so, :]
                vb[pd, h, :, do] = vb0[sp, h, :, so]
            elif td == ts == TAG_FP8:
                mx["k8"][pd, h, do, :] = old["k8"][sp, h, so, :]
                mx["v8"][pd, h, :, do] = old["v8"][sp, h, :, so]
                mx["k_scale"][pd, h, do] = old["k_scale"][sp, h, so]
                mx["v_scale"][pd, h, do] = old["v_scale"][sp, h, so]
            elif td == ts == TAG_INT4:
                mx["k4"][pd, h, do, :] = old["k4"][sp, h, so, :]
                w = vwork.setdefault((pd, h), np.zeros((kp.shape[3], b), dtype=np.int8))
                w[:, do] = unpack_values(old["v4"][sp, h])[:, so]
                mx["k4_scale"][pd, h, do] = old["k4_scale"][sp, h, so]
                mx["v4_scale"][pd, h, do] = old["v4_scale"][sp, h, so]
            else:
                assert td == TAG_BF16 and ts in (TAG_FP8, TAG_INT4)
                if ts == TAG_FP8:
                    kv = e4m3_decode(old["k8"][sp, h, so, :]) * float(old["k_scale"][sp, h, so])
                    vv = e4m3_decode(old["v8"][sp, h, :, so]) * float(old["v_scale"][sp, h, so])
                else:
                    kc = unpack_pairs(old["k4"][sp, h, so, :], axis=-1).astype(np.float64)
                    vc = unpack_values(old["v4"][sp, h])[:, so].astype(np.float64)
                    kv = kc * float(old["k4_scale"][sp, h, so])
                    vv = vc * float(old["v4_scale"][sp, h, so])
                kb[pd, h, do, :] = bf16_bits(kv)
                vb[pd, h, :, do] = bf16_bits(vv)
    for (pd, h), w in vwork.items():
        mx["v4"][pd, h] = pack_values(w)
    for dp, t in new_tag.items():
        tags[int(new_bt[dp])] = t


# ---------------------------------------------------------------------------- steps 5-8
def compact_or_grow(req_idx, a_short, a_long, ws_counts, n_cand, tau, k_loc, policy,
                    k_pool, v_pool, block_tables, n_pages, context_lens, refcount,
                    free_stack, free_top, page_size, policies=None, mixed=None):
    """Decision, allocation, selection and compaction for the boundary requests of one layer.

    State arrays (numpy) are updated in place: k_pool [N, H, b, d], v_pool [N, H, d, b],
    block_tables [B, max_pages], n_pages, context_lens, refcount, free_stack, free_top [1].
    `policies` optionally gives a per-request policy overriding `policy`. `mixed` (page_tag
    and the fp8 / INT4 pools of a mixed-precision cache, bf16 pools given as bit patterns)
    selects the mixed-precision compaction of _move_mixed.
    Returns decision [R] and kept_idx [R, H_kv, C_max] (-1 where unused).
    """
    dec, kept = compact_or_grow_layers(req_idx, [a_short], [a_long], [ws_counts], n_cand, tau,
                                       k_loc, policy, [k_pool], [v_pool], block_tables, n_pages,
                                       context_lens, refcount, free_stack, free_top, page_size,
                                       policies, None if mixed is None else [mixed])
    return dec, kept[0]


def _pop(free_stack, free_top):
    top = int(free_top[0]) - 1
    page = int(free_stack[top])
    free_stack[top] = -1
    free_top[0] = top
    return page


def compact_or_grow_layers(req_idx, a_short, a_long, ws_counts, n_cand, tau, k_loc, policy,
                           k_pools, v_pools, block_tables, n_pages, context_lens, refcount,
                           free_stack, free_top, page_size, policies=None, mixed_layers=None):
    """As compact_or_grow for L layers that share block tables and the page pool: a_short,
    a_long, ws_counts, k_pools, v_pools (and mixed_layers) are lists with one entry per layer.
    One decision per request from the mean over all layers and KV heads (Eq. 8); selection and
    compaction per layer. In a mixed-precision cache a request that must move tokens while one
    of its pages is released (in any layer) is left untouched (NO_PAGES): a page's precision
    is one tag for all its slots, so a released token could not stay masked among live ones.
    Returns decision [R] and a list of kept_idx [R, H_kv, C_max], one per layer."""
    b = page_size
    L = len(k_pools)
    R = len(req_idx)
    H = k_pools[0].shape[1]
    C_max = a_short[0].shape[2]
    max_pages = block_tables.shape[1]
    decision = np.full(R, -1, dtype=np.int64)
    kept_idx = [np.full((R, H, C_max), -1, dtype=np.int64) for _ in range(L)]
    releases = []
    for i, r in enumerate(req_idx):
        pol = policy if policies is None else policies[i]
        P = int(n_pages[r])
        ctx = int(context_lens[r])
        n = int(n_cand[i])
        assert n == candidate_count(ctx, b)
        R_n = ctx - n
        ws_r = np.concatenate([np.asarray(ws_counts[l][i]).reshape(-1, 2) for l in range(L)])
        action = primary_action(ws_r, n, tau, pol)
        code = COMPRESS
        if action == "grow":
            if int(free_top[0]) > 0 and P < max_pages:
                page = _pop(free_stack, free_top)
                block_tables[r, P] = page
                n_pages[r] = P + 1
                refcount[page] = 1
                decision[i] = GROW
                continue
            if n == 0:
                decision[i] = NO_PAGES
                continue
            code = GROW_FALLBACK_COMPRESS
        shrink = action == "shrink" and P >= 2 and (P - 1) * b >= MIN_CAPACITY
        if shrink:
            code = SHRINK
        keep_pages = P - 2 if shrink else P - 1
        K_t = min(n, max(0, keep_pages * b - R_n))
        E = n - K_t
        if E == 0:
            # nothing to evict: no token moves (a shrink still hands back the empty last page)
            for l in range(L):
                kept_idx[l][i, :, :n] = np.arange(n)
            if shrink:
                releases.append(int(block_tables[r, P - 1]))
                block_tables[r, P - 1] = -1
                n_pages[r] = P - 1
            decision[i] = code
            continue
        ctx_new = K_t + R_n
        n_dest = -(-ctx_new // b)
        if mixed_layers is not None and any(
                (np.asarray(m["page_tag"])[block_tables[r, :P]] == TAG_RELEASE).any()
                for m in mixed_layers):
            decision[i] = NO_PAGES
            continue
        shared = [j for j in range(n_dest) if refcount[block_tables[r, j]] > 1]
        if len(shared) > int(free_top[0]):
            decision[i] = NO_PAGES
            continue
        old_bt = block_tables[r].copy()
        for j in shared:
            page = _pop(free_stack, free_top)
            block_tables[r, j] = page
            refcount[page] = 1
            releases.append(int(old_bt[j]))
        # selection per layer and KV head, then move the tokens (read everything first)
        src_slots = np.arange(ctx)
        for l in range(L):
            srcs = []
            for h in range(H):
                s = np.maximum(np.asarray(a_short[l][i, h, :n], dtype=np.float64),
                               np.asarray(a_long[l][i, h, :n], dtype=np.float64))
                kept = select_kept(s, K_t, b, k_loc)
                kept_idx[l][i, h, :K_t] = kept
                src = np.concatenate([kept, src_slots[n:ctx]])
                srcs.append(src)
                if mixed_layers is not None:
                    continue
                sp, so = old_bt[src // b], src % b
                kv_k = k_pools[l][sp, h, so, :].copy()
                kv_v = v_pools[l][sp, h, :, so].copy()
                dst = np.arange(ctx_new)
                dp, do = block_tables[r][dst // b], dst % b
                k_pools[l][dp, h, do, :] = kv_k
                v_pools[l][dp, h, :, do] = kv_v
            if mixed_layers is not None:
                _move_mixed(k_pools[l], v_pools[l], mixed_layers[l], old_bt, block_tables[r],
                            srcs, min(shared) if shared else n_dest, ctx_new, b, P)
        if shrink:
            releases.append(int(old_bt[P - 1]))
            block_tables[r, P - 1] = -1
            n_pages[r] = P - 1
        context_lens[r] = ctx_new
        decision[i] = code
    for page in releases:
        refcount[page] -= 1
        if refcount[page] == 0:
            top = int(free_top[0])
            free_stack[top] = page
            free_top[0] = top + 1
    return decision, kept_idx
