"""Pins for GrowPage-Shrink (Eq. 13, App. H.1) and the multi-layer decision of Eq. 8 in the
boundary oracle: hand-worked decisions, and the invariants of a shrink and of a call over several
layers that share block tables."""
import numpy as np
import pytest

from oracle import boundary as ob
from oracle.summaries import update_query_summaries
from util import f64, golden_lines, npy, oracle_state
from workloads.configs import make_decode_case


def _cases():
    out = []
    for tok in golden_lines("shrink_cases.txt"):
        parts = " ".join(tok).split(";")
        action, n, tau, rows = (p.strip() for p in parts)
        ws = np.array([[int(x) for x in r.split(",")] for r in rows.split()])
        out.append((action, int(n), float(tau), ws))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}")
def test_shrink_decision_golden(case):
    action, n, tau, ws = case
    assert ob.primary_action(ws, n, tau, ob.POLICY_SHRINK) == action
    # the other policies never shrink
    assert ob.primary_action(ws, n, tau, ob.POLICY_AUTO) in ("grow", "compress")


def _state_and_scores(lens, seed=3):
    wl = make_decode_case(len(lens), 8, 2, 64, 16, lens, dtype="f32", seed=seed,
                          boundary=range(len(lens)))
    st = oracle_state(wl)
    qs = np.zeros((wl.qstate.shape[0], 2, wl.H_q, wl.d))
    for t in range(wl.q_hist.shape[0]):
        update_query_summaries(f64(wl.q_hist[t]), npy(wl.slot_ids), [t == 0] * wl.B, qs,
                               0.9, 0.999)
    req = list(range(wl.B))
    a_s, a_l, ws, nc = ob.score_and_working_set(
        f64(wl.q), qs, npy(wl.slot_ids), req, st["k_pool"], st["block_tables"],
        st["context_lens"], npy(wl.positions), wl.page_size, 10000.0, 0.99, wl.sm_scale)
    return wl, st, req, a_s, a_l, nc


def _check_pool(st, num_pages, B):
    held = {}
    for r in range(B):
        for j in range(int(st["n_pages"][r])):
            pg = int(st["block_tables"][r, j])
            held[pg] = held.get(pg, 0) + 1
    free = st["free_stack"][:int(st["free_top"][0])].tolist()
    assert len(set(free)) == len(free) and not (set(free) & set(held))
    assert set(free) | set(held) == set(range(num_pages))
    for pg in range(num_pages):
        assert st["refcount"][pg] == held.get(pg, 0)


def test_shrink_invariants_and_capacity_floor():
    # 75 pages (full), 65 pages (full: capacity after shrink exactly 1024), 64 pages (full:
    # 1008 < 1024 -> Compress & Hold), 70 pages with 4 tokens in the last one
    lens = [1200, 1040, 1024, 1108]
    wl, st, req, a_s, a_l, nc = _state_and_scores(lens)
    before = {k: v.copy() for k, v in st.items()}
    H = wl.H_kv
    ws = np.zeros((len(req), H, 2), dtype=np.int64)
    ws[:, :, 0], ws[:, :, 1] = 100, 200          # Delta far below -0.005 for every request
    dec, kept = ob.compact_or_grow(req, a_s, a_l, ws, nc, 0.0, wl.k_loc, ob.POLICY_SHRINK,
                                   st["k_pool"], st["v_pool"], st["block_tables"],
                                   st["n_pages"], st["context_lens"], st["refcount"],
                                   st["free_stack"], st["free_top"], wl.page_size)
    assert list(dec) == [ob.SHRINK, ob.SHRINK, ob.COMPRESS, ob.SHRINK]
    _check_pool(before, wl.num_pages, wl.B)
    _check_pool(st, wl.num_pages, wl.B)
    b = wl.page_size
    released = []
    for i, r in enumerate(req):
        P0, ctx0, n = int(before["n_pages"][r]), int(before["context_lens"][r]), int(nc[i])
        R_n = ctx0 - n
        if dec[i] == ob.SHRINK:
            K_t = (P0 - 2) * b - R_n
            assert st["n_pages"][r] == P0 - 1 and st["context_lens"][r] == (P0 - 2) * b
            assert st["block_tables"][r, P0 - 1] == -1
            released.append(int(before["block_tables"][r, P0 - 1]))
            assert n - K_t == b + R_n                 # two pages' worth at a full boundary
        else:
            K_t = (P0 - 1) * b - R_n
            assert st["n_pages"][r] == P0 and st["context_lens"][r] == (P0 - 1) * b
        assert st["n_pages"][r] * b >= ob.MIN_CAPACITY or dec[i] != ob.SHRINK  # capacity left
        for h in range(H):
            kk = kept[i, h, :K_t]
            assert np.all(np.diff(kk) > 0) and np.all(kept[i, h, K_t:] == -1)
            src = np.concatenate([kk, np.arange(n, ctx0)])
            for dst, sidx in enumerate(src):
                sp, so = before["block_tables"][r, sidx // b], sidx % b
                dp, do = st["block_tables"][r, dst // b], dst % b
                assert np.array_equal(st["k_pool"][dp, h, do], before["k_pool"][sp, h, so])
                assert np.array_equal(st["v_pool"][dp, h, :, do],
                                      before["v_pool"][sp, h, :, so])
    # the released last pages are back on the stack, in request order, after the free pages
    top0 = int(before["free_top"][0])
    assert st["free_stack"][top0:top0 + len(released)].tolist() == released


def test_layers_decision_is_the_mean_and_selection_is_per_layer():
    lens = [640, 500, 368]
    wl, st, req, a_s, a_l, nc = _state_and_scores(lens, seed=5)
    H = wl.H_kv
    # a second layer: other keys and values on the same pages (NaN slots stay NaN)
    k1 = -0.5 * st["k_pool"] + 0.25
    v1 = 2.0 * st["v_pool"] - 1.0
    qs = np.zeros((wl.qstate.shape[0], 2, wl.H_q, wl.d))
    for t in range(wl.q_hist.shape[0]):
        update_query_summaries(f64(wl.q_hist[t]), npy(wl.slot_ids), [t == 0] * wl.B, qs,
                               0.9, 0.999)
    a_s1, a_l1, _, nc1 = ob.score_and_working_set(
        f64(wl.q), qs, npy(wl.slot_ids), req, k1, st["block_tables"], st["context_lens"],
        npy(wl.positions), wl.page_size, 10000.0, 0.99, wl.sm_scale)
    assert np.array_equal(nc, nc1)
    # layer 0 says grow, layer 1 says compress more strongly: the mean compresses
    ws0 = np.zeros((len(req), H, 2), dtype=np.int64)
    ws1 = np.zeros_like(ws0)
    ws0[..., 0], ws0[..., 1] = 30, 20
    ws1[..., 0], ws1[..., 1] = 20, 31
    for i in range(len(req)):
        rows = np.concatenate([ws0[i], ws1[i]])
        assert ob.primary_action(rows, nc[i], 0.0, ob.POLICY_AUTO) == "compress"
        assert ob.primary_action(ws0[i], nc[i], 0.0, ob.POLICY_AUTO) == "grow"
    st1 = {k: v.copy() for k, v in st.items()}
    k_pools, v_pools = [st1["k_pool"], k1.copy()], [st1["v_pool"], v1.copy()]
    before_k = [p.copy() for p in k_pools]
    before_v = [p.copy() for p in v_pools]
    bt0 = st1["block_tables"].copy()
    dec, kept = ob.compact_or_grow_layers(req, [a_s, a_s1], [a_l, a_l1], [ws0, ws1], nc, 0.0,
                                          wl.k_loc, ob.POLICY_AUTO, k_pools, v_pools,
                                          st1["block_tables"], st1["n_pages"],
                                          st1["context_lens"], st1["refcount"],
                                          st1["free_stack"], st1["free_top"], wl.page_size)
    assert list(dec) == [ob.COMPRESS] * len(req)
    b = wl.page_size
    differs = False
    for i, r in enumerate(req):
        n, ctx0 = int(nc[i]), lens[i]
        K_t = (int(st["n_pages"][r]) - 1) * b - (ctx0 - n)
        for l in range(2):
            for h in range(H):
                kk = kept[l][i, h, :K_t]
                src = np.concatenate([kk, np.arange(n, ctx0)])
                for dst, sidx in enumerate(src):
                    sp, so = bt0[r, sidx // b], sidx % b
                    dp, do = st1["block_tables"][r, dst // b], dst % b
                    assert np.array_equal(k_pools[l][dp, h, do], before_k[l][sp, h, so])
                    assert np.array_equal(v_pools[l][dp, h, :, do], before_v[l][sp, h, :, so])
                differs |= not np.array_equal(kept[0][i, h], kept[1][i, h])
    assert differs                                  # the layers keep different tokens
    # one layer through the layered call is the single-layer call
    st2 = {k: v.copy() for k, v in st.items()}
    st3 = {k: v.copy() for k, v in st.items()}
    d2, k2 = ob.compact_or_grow(req, a_s, a_l, ws1, nc, 0.0, wl.k_loc, ob.POLICY_AUTO,
                                st2["k_pool"], st2["v_pool"], st2["block_tables"], st2["n_pages"],
                                st2["context_lens"], st2["refcount"], st2["free_stack"],
                                st2["free_top"], wl.page_size)
    d3, k3 = ob.compact_or_grow_layers(req, [a_s], [a_l], [ws1], nc, 0.0, wl.k_loc,
                                       ob.POLICY_AUTO, [st3["k_pool"]], [st3["v_pool"]],
                                       st3["block_tables"], st3["n_pages"], st3["context_lens"],
                                       st3["refcount"], st3["free_stack"], st3["free_top"],
                                       wl.page_size)
    assert np.array_equal(d2, d3) and np.array_equal(k2, k3[0])
    for k in st2:
        assert np.array_equal(st2[k], st3[k], equal_nan=True), k
