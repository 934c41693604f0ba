"""Pins for GrowPage's boundary-pass oracle: calibration, RoPE, working set, decision,
selection, allocation and compaction (GrowPage Sec. 3, Sec. 4.2, App. C, App. E)."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as oatt
from oracle import boundary as ob
from oracle.summaries import update_query_summaries
from workloads import make_workload
from util import f64, golden_lines, npy, oracle_state


# ------------------------------------------------------------------ calibration and RoPE
def test_calibration_matches_current_rms():
    rng = np.random.default_rng(0)
    q, qb = rng.standard_normal(64), rng.standard_normal(64) * 0.01
    qt = ob.calibrate(q, qb)
    assert abs(ob.rms(qt) - ob.rms(q)) < 1e-12
    assert np.allclose(qt / np.linalg.norm(qt), qb / np.linalg.norm(qb), atol=1e-12)
    assert np.all(ob.calibrate(q, np.zeros(64)) == 0)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for pos in (0, 1, 4097, 32767):
        assert abs(np.linalg.norm(ob.rope(q, pos, 10000.0)) - np.linalg.norm(q)) < 1e-9
    d1 = ob.rope(q, 900, 1e4) @ ob.rope(k, 300, 1e4)
    d2 = ob.rope(q, 1600, 1e4) @ ob.rope(k, 1000, 1e4)
    assert abs(d1 - d2) < 1e-9
    assert np.array_equal(ob.rope(q, 0, 1e4), q)
    assert np.array_equal(ob.rope(q, 123, 0.0), q)


def test_rope_rotates_pairs_by_hand():
    # d = 4: pair (0, 2) turns by pos * 1, pair (1, 3) by pos * theta^(-1/2)
    x = np.array([1.0, 0.0, 0.0, 1.0])
    y = ob.rope(x, 1, 100.0)
    assert np.allclose(y, [math.cos(1), -math.sin(0.1), math.sin(1), math.cos(0.1)], atol=1e-15)


# ------------------------------------------------------------------ working set (Eq. 2 / 7)
def test_working_set_golden():
    lines = list(golden_lines("working_set_cases.txt"))
    w = np.array([float(x) for x in lines[0][1:]])
    for p, k in lines[1:]:
        assert ob.working_set_size(w, float(p)) == int(k)
        assert ob.working_set_size(w.astype(np.float32), float(p)) == int(k)


def test_working_set_closed_forms():
    n = 64
    uni = np.full(n, 1.0 / n)
    for p in (0.1, 0.5, 0.9, 0.99, 1.0):
        assert ob.working_set_size(uni, p) == math.ceil(Fraction(p) * n)
    dom = np.concatenate([[0.995], np.full(n - 1, 0.005 / (n - 1))])
    assert ob.working_set_size(dom, 0.99) == 1
    # full retention: every weight positive and p = total mass -> K = |C|
    w = np.array([2.0 ** -(i + 1) for i in range(20)] + [2.0 ** -20])
    assert Fraction(float(w.sum())) == 1
    assert ob.working_set_size(w, 1.0) == len(w)
    assert ob.working_set_size(np.zeros(0), 0.9) == 0
    # mass below p everywhere -> K = |C|
    assert ob.working_set_size(np.full(10, 0.05), 0.99) == 10


def test_working_set_exact_near_threshold():
    # float32 0.3 is slightly above 0.3 and float64 0.3 slightly below; exactness decides.
    w32 = np.array([0.5, 0.3, 0.2], dtype=np.float32)
    assert Fraction(float(w32[0])) + Fraction(float(w32[1])) >= Fraction(0.8)
    assert ob.working_set_size(w32, 0.8) == 2
    w64 = np.array([0.5, 0.3, 0.2])
    assert Fraction(0.5) + Fraction(0.3) < Fraction(0.8)
    assert ob.working_set_size(w64, 0.8) == 3


@pytest.mark.parametrize("seed", range(6))
def test_working_set_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = 10
    z = rng.standard_normal(n) * (seed + 1)
    a = np.exp(z - z.max())
    a = (a / a.sum()).astype(np.float32)
    for p in (0.3, 0.6, 0.9, 0.99):
        best = None
        for k in range(1, n + 1):
            for S in itertools.combinations(range(n), k):
                if sum(Fraction(float(a[i])) for i in S) >= Fraction(p):
                    best = k
                    break
            if best:
                break
        assert ob.working_set_size(a, p) == (best or n)


def test_theorem_3_1_tight_construction():
    # App. C: with v_i = -Vmax u on S and +Vmax u off S the error equals 2 Vmax (1 - m(S)).
    rng = np.random.default_rng(3)
    a = rng.dirichlet(np.ones(12))
    S = np.argsort(-a)[:ob.working_set_size(a, 0.8)]
    m = a[S].sum()
    u = rng.standard_normal(5)
    u /= np.linalg.norm(u)
    vmax = 2.5
    v = np.tile(vmax * u, (12, 1))
    v[S] = -vmax * u
    o = a @ v
    o_hat = (a[S] / m) @ v[S]
    assert abs(np.linalg.norm(o - o_hat) - 2 * vmax * (1 - m)) < 1e-12
    # and no admissible value set does worse (Eq. 5 upper bound)
    for _ in range(200):
        v = rng.standard_normal((12, 5))
        v *= vmax / np.maximum(np.linalg.norm(v, axis=1, keepdims=True), vmax)
        err = np.linalg.norm(a @ v - (a[S] / m) @ v[S])
        assert err <= 2 * vmax * (1 - m) + 1e-12
    # Eq. 3 with S = everything: renormalised output equals the full output
    v = rng.standard_normal((12, 5))
    assert np.allclose((a / a.sum()) @ v, a @ v, atol=1e-12)


# ------------------------------------------------------------------ scores
def test_scores_are_distributions_and_views_agree_when_equal():
    wl = make_workload("tiny", "small")
    st = np.zeros((512, 2, wl.H_q, wl.d))
    q = f64(wl.q)
    update_query_summaries(q, npy(wl.slot_ids), [1] * wl.B, st, 0.9, 0.999)  # both = q_t
    a_s, a_l, ws, nc = ob.score_and_working_set(
        q, st, npy(wl.slot_ids), [0, 1], f64(wl.k_pool), npy(wl.block_tables),
        npy(wl.context_lens), npy(wl.positions), wl.page_size, 1e4, 0.9, wl.sm_scale)
    assert list(nc) == [192, 320]
    for i, n in enumerate(nc):
        assert np.allclose(a_s[i, :, :n].sum(axis=1), 1.0, atol=1e-12)
        assert np.all(a_s[i, :, n:] == 0)
    assert np.array_equal(a_s, a_l) and np.array_equal(ws[..., 0], ws[..., 1])
    # equal summaries -> Delta = 0 -> compress; the inverse policy grows
    for i in range(2):
        assert not ob.wants_grow(ws[i], nc[i], 0.0, ob.POLICY_AUTO)
        assert ob.wants_grow(ws[i], nc[i], 0.0, ob.POLICY_INVERSE)


def test_score_matches_single_head_softmax_by_hand():
    # G = 1, no RoPE, qbar already at the RMS of q_t: plain softmax of the candidate keys.
    rng = np.random.default_rng(5)
    d, n = 8, 40
    keys = rng.standard_normal((1, n, d))
    q = rng.standard_normal((1, d))
    qbar = np.stack([q * 3, -q])[:, :]                 # calibration undoes the factor 3
    a = ob.score_request(q, qbar, 7, keys, 0.0, 0.5, 1)
    z = keys[0] @ q[0] * 0.5
    ref = np.exp(z - z.max()) / np.exp(z - z.max()).sum()
    assert np.allclose(a[0, 0], ref, atol=1e-14)
    zl = -z
    refl = np.exp(zl - zl.max()) / np.exp(zl - zl.max()).sum()
    assert np.allclose(a[1, 0], refl, atol=1e-14)


# ------------------------------------------------------------------ decision
def test_score_gqa_golden():
    """Hand-worked scores with G = 2 (tests/golden/score_gqa.txt): each KV head's weights are the
    mean of its own query heads' softmax distributions."""
    from fractions import Fraction
    rows = {r[0]: r[1:] for r in golden_lines("score_gqa.txt")}
    b, d, H_q = 16, 2, 4
    ln4, ln9 = math.log(4.0), math.log(9.0)
    q = np.array([[[0.0, 0.0], [ln4, 0.0], [0.0, ln9], [0.0, 0.0]]])
    qstate = np.zeros((1, 2, H_q, d))
    qstate[0, 0] = q[0]
    qstate[0, 1] = 3.0 * q[0]
    qstate[0, :, 0] = qstate[0, :, 3] = (1.0, 1.0)    # q_t = 0 there: the calibrated summary is 0
    k_pool = np.zeros((2, 2, b, d))
    k_pool[0, 0, 0], k_pool[0, 0, 1], k_pool[0, 0, 2:] = (1, 0), (0, 1), (0, -1)
    k_pool[0, 1, 0], k_pool[0, 1, 1], k_pool[0, 1, 2:] = (0, 1), (0, 0), (1, 0)
    a_s, a_l, ws, nc = ob.score_and_working_set(q, qstate, [0], [0], k_pool, np.array([[0, 1]]),
                                                [20], [19], b, 0.0, 0.2, 1.0)
    assert nc.tolist() == [16]
    for h in range(2):
        fr = [float(Fraction(x)) for x in rows[f"a_h{h}"]]
        expect = np.array(fr[:2] + [fr[2]] * 14)
        assert np.allclose(a_s[0, h, :16], expect, rtol=1e-12, atol=0)
        assert np.allclose(a_l[0, h, :16], expect, rtol=1e-12, atol=0)
    assert ws[0, :, 0].tolist() == [int(x) for x in rows["ws"]]
    assert ws[0, :, 1].tolist() == [int(x) for x in rows["ws"]]


def test_decision_golden():
    for row in golden_lines("decision_cases.txt"):
        ks0, kl0, ks1, kl1, n, tau, pol, dec = row
        ws = np.array([[int(ks0), int(kl0)], [int(ks1), int(kl1)]])
        assert ob.wants_grow(ws, int(n), float(tau), int(pol)) == bool(int(dec)), row


def test_decision_forced_and_empty():
    ws = np.array([[1, 100]])
    assert ob.wants_grow(ws, 10, 0.0, ob.POLICY_FORCE_GROW)
    assert not ob.wants_grow(np.array([[100, 1]]), 10, 0.0, ob.POLICY_FORCE_COMPRESS)
    assert ob.wants_grow(np.zeros((1, 2), int), 0, 0.0, ob.POLICY_AUTO)


# ------------------------------------------------------------------ selection (Eq. 9, 10)
def test_selection_golden():
    rows = list(golden_lines("selection_cases.txt"))
    aS = np.array([float(x) for x in rows[0][1:]])
    aL = np.array([float(x) for x in rows[1][1:]])
    b, kloc = int(rows[2][1]), int(rows[3][1])
    s = np.maximum(aS, aL)
    for row in rows[4:]:
        K = int(row[1])
        kept = [int(x) for x in row[3:]]
        assert ob.select_kept(s, K, b, kloc).tolist() == kept


@pytest.mark.parametrize("seed", range(8))
def test_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    b, kloc, n = 4, 1 + seed % 2, 12
    s = rng.integers(0, 5, size=n).astype(np.float64) / 8    # many ties
    key = lambda i: (-s[i], i)                                 # noqa: E731
    loc = set()
    for j in range(0, n, b):
        loc |= set(sorted(range(j, min(n, j + b)), key=key)[:kloc])
    for K in range(0, n + 1):
        got = ob.select_kept(s, K, b, kloc).tolist()
        if K >= n:
            assert got == list(range(n))
            continue
        # brute force: among all K-subsets containing S_loc (or, if S_loc is too large, all
        # K-subsets), take the one whose members sorted by key come first lexicographically
        pool = [S for S in itertools.combinations(range(n), K)
                if (len(loc) >= K or loc <= set(S))]
        best = min(pool, key=lambda S: sorted(key(i) for i in S
                                               if len(loc) >= K or i not in loc))
        assert got == sorted(best)


def test_selection_paper_scale_closed_form():
    """256-token pages with a 64-token local quota (GrowPage's default runs, App. D.2). With scores
    strictly decreasing in the token index, each page's quota is its first 64 tokens and the
    global fill takes the lowest remaining indices; strictly increasing scores mirror it."""
    b, kloc, n = 256, 64, 4 * 256
    K = 3 * 256                                   # P = 5 full pages: (P - 1) b - |R| = 768
    dec = ob.select_kept(np.arange(n, 0, -1, dtype=np.float64), K, b, kloc)
    # non-quota tokens: 192 per page; the 256 worst are page 3's 192 and page 2's last 64
    assert dec.tolist() == list(range(0, 704)) + list(range(768, 832))
    inc = ob.select_kept(np.arange(1, n + 1, dtype=np.float64), K, b, kloc)
    # mirrored: page 0's 192 non-quota tokens and page 1's first 64 go
    assert inc.tolist() == list(range(192, 256)) + list(range(320, 1024))
    # every page keeps at least its quota
    for kept in (dec, inc):
        assert all(np.sum((kept >= j) & (kept < j + b)) >= kloc for j in range(0, n, b))


# ------------------------------------------------------------------ allocation + compaction
def _run_boundary(wl, policies=None, free_top=None):
    st = oracle_state(wl)
    if free_top is not None:
        st["free_top"][0] = free_top
    qs = np.zeros((512, 2, wl.H_q, wl.d))
    for t in range(wl.q_hist.shape[0]):
        update_query_summaries(f64(wl.q_hist[t]), npy(wl.slot_ids), [t == 0] * wl.B, qs,
                               wl.beta_s, wl.beta_l)
    update_query_summaries(f64(wl.q), npy(wl.slot_ids), [0] * wl.B, qs, wl.beta_s, wl.beta_l)
    req = npy(wl.req_idx).tolist()
    a_s, a_l, ws, nc = ob.score_and_working_set(
        f64(wl.q), qs, npy(wl.slot_ids), req, st["k_pool"], st["block_tables"],
        st["context_lens"], npy(wl.positions), wl.page_size, wl.rope_theta, wl.p, wl.sm_scale)
    before = {k: v.copy() for k, v in st.items()}
    dec, kept = ob.compact_or_grow(req, a_s, a_l, ws, nc, wl.tau, wl.k_loc, ob.POLICY_AUTO,
                                   st["k_pool"], st["v_pool"], st["block_tables"],
                                   st["n_pages"], st["context_lens"], st["refcount"],
                                   st["free_stack"], st["free_top"], wl.page_size,
                                   policies=policies)
    return before, st, dec, kept, req, (a_s, a_l, ws, nc)


def _check_pool_invariants(wl, st, check_free=True):
    held = {}
    for r in range(wl.B):
        for j in range(int(st["n_pages"][r])):
            pg = int(st["block_tables"][r, j])
            held[pg] = held.get(pg, 0) + 1
    top = int(st["free_top"][0])
    free = st["free_stack"][:top].tolist()
    assert len(set(free)) == len(free)
    assert not (set(free) & set(held))
    if check_free:
        assert set(free) | set(held) == set(range(wl.num_pages))      # page conservation
    for pg in range(wl.num_pages):
        assert st["refcount"][pg] == held.get(pg, 0)                 # refcounts = references


@pytest.mark.parametrize("cfg,page_size", [("tiny", 16), ("long_reasoning_d64", 16), ("prefix_shared", 16), ("long_reasoning_d64", 256),
                                            ("prefix_shared", 64), ("tiny", 128)])
def test_compaction_invariants(cfg, page_size):
    wl = make_workload(cfg, "small", page_size=page_size)
    pol = wl.req_policy if cfg == "prefix_shared" else None
    before, st, dec, kept, req, (a_s, a_l, ws, nc) = _run_boundary(wl, policies=pol)
    _check_pool_invariants(wl, before)
    _check_pool_invariants(wl, st)
    b = wl.page_size
    top = int(before["free_top"][0])          # pops come off the LIFO stack in request order
    for i, r in enumerate(req):
        P0, ctx0 = int(before["n_pages"][r]), int(before["context_lens"][r])
        if dec[i] == ob.GROW:
            assert st["n_pages"][r] == P0 + 1 and st["context_lens"][r] == ctx0
            assert st["block_tables"][r, P0] == before["free_stack"][top - 1]
            top -= 1
            continue
        for j in range(P0):
            if st["block_tables"][r, j] != before["block_tables"][r, j]:
                assert st["block_tables"][r, j] == before["free_stack"][top - 1]
                top -= 1
        assert dec[i] in (ob.COMPRESS, ob.GROW_FALLBACK_COMPRESS)
        n = int(nc[i])
        R_n = ctx0 - n
        # the protected tokens are the whole last page, also where it is longer than the
        # 16-token recent window (b = 256): none of them is a candidate
        assert R_n == ctx0 - (-(-ctx0 // b) - 1) * b and 0 < R_n <= b
        K_t = min(n, (P0 - 1) * b - R_n)
        assert st["context_lens"][r] == K_t + R_n == (P0 - 1) * b
        assert st["n_pages"][r] == P0
        for h in range(wl.H_kv):
            kk = kept[i, h, :K_t]
            assert np.all(np.diff(kk) > 0) and np.all(kept[i, h, K_t:] == -1)
            src = np.concatenate([kk, np.arange(n, ctx0)])
            for dst, sidx in enumerate(src):               # kept K/V bit-identical
                sp, so = before["block_tables"][r, sidx // b], sidx % b
                dp, do = st["block_tables"][r, dst // b], dst % b
                assert np.array_equal(st["k_pool"][dp, h, do], before["k_pool"][sp, h, so])
                assert np.array_equal(st["v_pool"][dp, h, :, do], before["v_pool"][sp, h, :, so])
    if cfg == "prefix_shared":
        shared = before["block_tables"][0, :wl.shared_pages]
        assert np.array_equal(st["k_pool"][shared], before["k_pool"][shared])
        assert np.array_equal(st["v_pool"][shared], before["v_pool"][shared])
        for i, r in enumerate(req):
            if dec[i] != ob.GROW:
                assert np.all(st["refcount"][st["block_tables"][r, :wl.shared_pages]] == 1)


def test_grow_leaves_attention_bit_identical():
    wl = make_workload("prefix_shared", "small")
    before, st, dec, kept, req, _ = _run_boundary(wl, policies=[ob.POLICY_FORCE_GROW] * 2)
    assert list(dec) == [ob.GROW, ob.GROW]
    args = dict(page_size=wl.page_size, sm_scale=wl.sm_scale)
    o1, _ = oatt.paged_decode_attn(f64(wl.q), before["k_pool"], before["v_pool"],
                                   before["block_tables"], before["context_lens"], **args)
    o2, _ = oatt.paged_decode_attn(f64(wl.q), st["k_pool"], st["v_pool"], st["block_tables"],
                                   st["context_lens"], **args)
    assert np.array_equal(o1, o2)


def test_empty_pool_fallback_and_no_pages():
    wl = make_workload("prefix_shared", "small")
    # no free page: forced grow falls back to compress, which needs replacement pages for the
    # shared prefix -> NO_PAGES and the request is untouched
    before, st, dec, kept, req, _ = _run_boundary(wl, policies=[ob.POLICY_FORCE_GROW] * 2,
                                                  free_top=0)
    assert list(dec) == [ob.NO_PAGES, ob.NO_PAGES]
    for k in ("block_tables", "n_pages", "context_lens", "refcount", "free_top"):
        assert np.array_equal(st[k], before[k])
    assert np.array_equal(st["k_pool"], before["k_pool"], equal_nan=True)
    wl1 = make_workload("tiny", "small")
    before, st, dec, kept, req, _ = _run_boundary(wl1, policies=[ob.POLICY_FORCE_GROW] * 2,
                                                  free_top=0)
    assert list(dec) == [ob.GROW_FALLBACK_COMPRESS] * 2
    _check_pool_invariants(wl1, st, check_free=False)
