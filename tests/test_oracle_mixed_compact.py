"""CPU pins of the oracle's compaction of mixed-precision pages (GrowPage Sec. 3.3 compaction
over PASK App. B.2 / B.5 page formats) and of its bf16 rounding.

Hand-derived expectations: which tag every destination page takes when the evicted tokens are
placed by hand, that tokens moving between pages of one precision keep their codes and row
scales bit for bit, that a page fed from two precisions holds each token's dequantised value
rounded once to bf16, that a request holding a released page is left alone, and that a mixed
cache whose pages are all bf16 compacts exactly like a uniform bf16 cache."""
import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle import boundary as ob
from oracle.int4 import pack_values
from workloads.configs import make_decode_case

F8, BF, I4, REL = ob.TAG_FP8, ob.TAG_BF16, ob.TAG_INT4, ob.TAG_RELEASE


def test_bf16_bits_hand_values():
    cases = [(1.0, 0x3F80), (1.0 + 2.0 ** -8, 0x3F80),             # tie -> even (down)
             (1.0 + 3 * 2.0 ** -8, 0x3F82),                         # tie -> even (up)
             (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),                # above the tie: rounding
             # through float32 first would lose the 2^-30 and round down to 0x3F80
             (-1.5, 0xBFC0), (0.0, 0x0000), (-0.0, 0x8000),
             (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),          # subnormal tie -> even
             (3 * 2.0 ** -134, 0x0002), (2.0 ** -126, 0x0080)]
    for x, bits in cases:
        assert int(ob.bf16_bits(np.array([x]))[0]) == bits, (x, hex(bits))


def test_bf16_bits_matches_torch_on_float32_values():
    # float32 inputs round once on either side, so torch's float32 -> bfloat16 (nearest, ties
    # to even) is the reference there
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ob.bf16_bits(x.astype(np.float64)), ref)


def _mixed_case(tags_req, b=16, d=64, H=2, seed=3):
    """One boundary request whose pages carry the given tags, random codes and scales."""
    lens = [len(tags_req) * b]
    wl = make_decode_case(1, 2 * H, H, d, b, lens, seed=seed, boundary=[0])
    rng = np.random.default_rng(seed)
    P = wl.num_pages
    k8 = rng.integers(0, 256, size=(P, H, b, d)).astype(np.uint8)
    v8 = rng.integers(0, 256, size=(P, H, d, b)).astype(np.uint8)
    for a in (k8, v8):
        a[(a & 0x7F) == 0x7F] = 0x3C                             # no NaN codes
    sc = lambda: rng.uniform(0.01, 3.0, size=(P, H, b)).astype(np.float32)  # noqa: E731
    k4c = rng.integers(-7, 8, size=(P, H, b, d))
    from oracle.int4 import pack_pairs
    mx = dict(page_tag=np.full(P, BF, dtype=np.uint8), k8=k8, v8=v8, k_scale=sc(), v_scale=sc(),
              k4=pack_pairs(k4c, axis=-1),
              v4=pack_values(rng.integers(-7, 8, size=(P, H, d, b))),
              k4_scale=rng.uniform(0.01, 2.0, size=(P, H, b)).astype(np.float16).astype(np.float64),
              v4_scale=rng.uniform(0.01, 2.0, size=(P, H, b)).astype(np.float16).astype(np.float64))
    bt = wl.block_tables.numpy().astype(np.int64)
    for j, t in enumerate(tags_req):
        mx["page_tag"][bt[0, j]] = t
    kbits = wl.k_pool.view(torch.int16).numpy().copy()
    vbits = wl.v_pool.view(torch.int16).numpy().copy()
    return wl, mx, kbits, vbits


def _state(wl):
    return dict(block_tables=wl.block_tables.numpy().astype(np.int64).copy(),
                n_pages=wl.n_pages.numpy().astype(np.int64).copy(),
                context_lens=wl.context_lens.numpy().astype(np.int64).copy(),
                refcount=wl.refcount.numpy().astype(np.int64).copy(),
                free_stack=wl.free_stack.numpy().astype(np.int64).copy(),
                free_top=wl.free_top.numpy().astype(np.int64).copy())


def _values(kbits, vbits, mx, st, b):
    """Dequantised K/V [H, n, d] of request 0 (released pages dropped) and their slots."""
    kf = (kbits.astype(np.int64) << 16).astype(np.uint32).view(np.float32)
    vf = (vbits.astype(np.int64) << 16).astype(np.uint32).view(np.float32)
    return oatt.gather_request_kv(0, kf, vf, st["block_tables"], st["context_lens"], b,
                                  mx["page_tag"], mx["k8"], mx["v8"], mx["k_scale"],
                                  mx["v_scale"], mx["k4"], mx["v4"], mx["k4_scale"],
                                  mx["v4_scale"])


def _compress(wl, mx, kbits, vbits, st, evict, k_loc=0):
    b = wl.page_size
    n = ob.candidate_count(int(st["context_lens"][0]), b)
    s = np.ones((1, wl.H_kv, n), dtype=np.float32)
    s[:, :, evict] = 0.5
    nc = np.array([n])
    ws = np.zeros((1, wl.H_kv, 2), dtype=np.int64)
    return ob.compact_or_grow([0], s.astype(np.float64), s.astype(np.float64), ws, nc, 0.0,
                              k_loc, ob.POLICY_FORCE_COMPRESS, kbits, vbits,
                              st["block_tables"], st["n_pages"], st["context_lens"],
                              st["refcount"], st["free_stack"], st["free_top"], b, mixed=mx)


@pytest.mark.parametrize("evict,expect,n_conv", [
    # the whole first page goes: every destination page is the next old page
    (list(range(16)), [F8, F8, I4, I4, BF], 0),
    # half of page 0 and half of page 2 go: page 0 mixes bf16 + fp8 -> bf16 (its last 8
    # tokens come from the fp8 page 1); page 1 reads fp8 pages only; pages 2 and 3 read INT4
    # pages only; page 4 reads the bf16 last page
    (list(range(8)) + list(range(40, 48)), [BF, F8, I4, I4, BF], 8),
])
def test_destination_tags_by_hand(evict, expect, n_conv):
    tags = [BF, F8, F8, I4, I4, BF]
    wl, mx, kb, vb = _mixed_case(tags)
    st = _state(wl)
    k0, v0, slots0 = _values(kb, vb, {k: np.copy(v) for k, v in mx.items()}, _state(wl), 16)
    before_tags = mx["page_tag"].copy()
    bt = st["block_tables"].copy()
    dec, kept = _compress(wl, mx, kb, vb, st, evict)
    assert list(dec) == [ob.COMPRESS]
    assert [int(mx["page_tag"][bt[0, j]]) for j in range(5)] == expect
    assert st["context_lens"][0] == 5 * 16
    k1, v1, slots1 = _values(kb, vb, mx, st, 16)
    assert np.array_equal(slots1, np.arange(80))
    src = np.array([t for t in range(96) if t not in set(evict)])   # kept, then the last page
    old_tag_of = np.array([before_tags[bt[0, t // 16]] for t in src])
    new_tag_of = np.array([expect[j // 16] for j in range(80)])
    carried = old_tag_of == new_tag_of
    # a token that keeps its precision keeps its exact value; one that lands in a bf16 page
    # from an fp8 or INT4 page holds its value rounded once to bf16
    for h in range(wl.H_kv):
        assert np.array_equal(k1[h][carried], k0[h][src[carried]])
        assert np.array_equal(v1[h][carried], v0[h][src[carried]])
        conv = ~carried
        rk = ob.bf16_bits(k0[h][src[conv]]).astype(np.uint32) << 16
        rv = ob.bf16_bits(v0[h][src[conv]]).astype(np.uint32) << 16
        assert np.array_equal(k1[h][conv].astype(np.float32).view(np.uint32), rk)
        assert np.array_equal(v1[h][conv].astype(np.float32).view(np.uint32), rv)
        assert conv.sum() == n_conv


def test_one_precision_moves_codes_and_scales_bit_for_bit():
    tags = [F8] * 5 + [I4]
    wl, mx, kb, vb = _mixed_case(tags, seed=5)
    st = _state(wl)
    bt = st["block_tables"].copy()
    k8_0, ks_0 = mx["k8"].copy(), mx["k_scale"].copy()
    rng = np.random.default_rng(1)
    evict = sorted(rng.choice(80, size=16, replace=False).tolist())
    dec, _ = _compress(wl, mx, kb, vb, st, evict)
    assert list(dec) == [ob.COMPRESS]
    keep = [t for t in range(80) if t not in set(evict)]
    for j, t in enumerate(keep):
        dp, sp = bt[0, j // 16], bt[0, t // 16]
        if mx["page_tag"][dp] == F8:
            assert np.array_equal(mx["k8"][dp, :, j % 16], k8_0[sp, :, t % 16])
            assert np.array_equal(mx["k_scale"][dp, :, j % 16], ks_0[sp, :, t % 16])
    # every eviction lies before slot 80, so destination pages 0..3 read fp8 pages only and
    # the last one is exactly the old INT4 last page
    assert [int(mx["page_tag"][bt[0, j]]) for j in range(5)] == [F8] * 4 + [I4]


def test_released_page_leaves_request_untouched():
    wl, mx, kb, vb = _mixed_case([BF, REL, F8, F8, BF], seed=7)
    st = _state(wl)
    before = {k: v.copy() for k, v in st.items()}
    kb0, tags0 = kb.copy(), mx["page_tag"].copy()
    dec, kept = _compress(wl, mx, kb, vb, st, list(range(16)))
    assert list(dec) == [ob.NO_PAGES]
    for k in before:
        assert np.array_equal(st[k], before[k])
    assert np.array_equal(kb, kb0) and np.array_equal(mx["page_tag"], tags0)


def test_all_bf16_mixed_equals_uniform():
    wl, mx, kb, vb = _mixed_case([BF] * 6, seed=9)
    st1, st2 = _state(wl), _state(wl)
    kb2, vb2 = kb.copy(), vb.copy()
    rng = np.random.default_rng(2)
    evict = sorted(rng.choice(80, size=16, replace=False).tolist())
    _compress(wl, mx, kb, vb, st1, evict)
    n = 80
    s = np.ones((1, wl.H_kv, n))
    s[:, :, evict] = 0.5
    ob.compact_or_grow([0], s, s, np.zeros((1, wl.H_kv, 2), np.int64), np.array([n]), 0.0, 0,
                       ob.POLICY_FORCE_COMPRESS, kb2, vb2, st2["block_tables"], st2["n_pages"],
                       st2["context_lens"], st2["refcount"], st2["free_stack"], st2["free_top"],
                       16)
    assert np.array_equal(kb, kb2) and np.array_equal(vb, vb2)
    assert (mx["page_tag"][st1["block_tables"][0, :5]] == BF).all()


def test_mixed_scores_equal_dequantised_pages_and_released_deleted():
    """Scores over a mixed cache equal the scores over a float cache holding each page's
    dequantised values with the released pages deleted from the block table."""
    tags = [F8, REL, I4, BF, REL, F8, BF]
    wl, mx, kb, vb = _mixed_case(tags, seed=11)
    b, H, d = 16, wl.H_kv, wl.d
    st = _state(wl)
    kf = (kb.astype(np.int64) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    qs = np.random.default_rng(4).standard_normal((wl.qstate.shape[0], 2, wl.H_q, d))
    q = wl.q.double().numpy()
    args = dict(rope_theta=10000.0, p=0.9, sm_scale=d ** -0.5)
    a_s, a_l, ws, nc = ob.score_and_working_set(q, qs, wl.slot_ids.numpy(), [0], kf,
                                                st["block_tables"], st["context_lens"],
                                                [int(st["context_lens"][0]) - 1], b, mixed=mx,
                                                **args)
    # the same keys dequantised into a float pool, released pages dropped from the table
    k_all, _, slots = _values(kb, vb, mx, st, b)            # visible tokens only, in order
    n_vis = k_all.shape[1]
    pool = k_all.transpose(1, 0, 2).reshape(n_vis // b, b, H, d).transpose(0, 2, 1, 3)
    bt2 = np.arange(n_vis // b)[None, :]
    r_s, r_l, rws, rnc = ob.score_and_working_set(q, qs, wl.slot_ids.numpy(), [0], pool, bt2,
                                                  [n_vis], [int(st["context_lens"][0]) - 1],
                                                  b, **args)
    vis_c = slots[slots < nc[0]]                             # visible candidates
    assert rnc[0] == len(vis_c)
    for a, r in ((a_s, r_s), (a_l, r_l)):
        assert np.allclose(a[0][:, vis_c], r[0][:, :len(vis_c)], rtol=1e-12, atol=0)
        mask = np.ones(nc[0], dtype=bool)
        mask[vis_c] = False
        assert (a[0][:, :nc[0]][:, mask] == 0).all()
    assert np.array_equal(ws, rws)


def test_destination_tag_from_supplying_pages_not_their_range():
    """A Shrink evicts 2b tokens: here all of page 1 (bf16) and half of pages 0 and 2 (fp8), the
    same in every head, with no per-page quota (k_loc = 0). Destination page 0 then receives
    slots 0..7 of page 0 and slots 32..39 of page 2: both fp8, so it stays an fp8 page and its
    tokens keep their codes and scales, although the bf16 page 1 lies between its suppliers."""
    tags = [F8, BF] + [F8] * 63 + [BF]                # 66 pages, the last one the recent page
    wl, mx, kb, vb = _mixed_case(tags, seed=13)
    st = _state(wl)
    bt = st["block_tables"].copy()
    k8_0, ks_0 = mx["k8"].copy(), mx["k_scale"].copy()
    n = 65 * 16
    evict = list(range(8, 32)) + list(range(40, 48))
    s = np.ones((1, wl.H_kv, n))
    s[:, :, evict] = 0.5
    ws = np.zeros((1, wl.H_kv, 2), dtype=np.int64)
    ws[..., 1] = n                                    # Delta = -1 < -0.005: shrink
    dec, kept = ob.compact_or_grow([0], s, s, ws, np.array([n]), 0.0, 0, ob.POLICY_SHRINK, kb,
                                   vb, st["block_tables"], st["n_pages"], st["context_lens"],
                                   st["refcount"], st["free_stack"], st["free_top"], 16, mixed=mx)
    assert list(dec) == [ob.SHRINK]
    assert st["context_lens"][0] == 64 * 16
    kept_slots = [t for t in range(n) if t not in set(evict)]
    assert np.array_equal(kept[0, 0, :n - 32], kept_slots)
    assert int(mx["page_tag"][bt[0, 0]]) == F8        # the range rule would make it bf16
    src = kept_slots[:16]
    assert src == list(range(8)) + list(range(32, 40))
    for j, t in enumerate(src):
        assert np.array_equal(mx["k8"][bt[0, 0], :, j], k8_0[bt[0, t // 16], :, t % 16])
        assert np.array_equal(mx["k_scale"][bt[0, 0], :, j], ks_0[bt[0, t // 16], :, t % 16])
    # destination page 1 reads page 3 only; the last kept page is the old recent (bf16) page
    assert int(mx["page_tag"][bt[0, 1]]) == F8
    assert int(mx["page_tag"][bt[0, 63]]) == BF


def test_retagging_a_mixed_workload_leaves_no_poison_in_context():
    """Re-tagging a workload that is already mixed (as the boundary-pass benchmark does): every
    in-context token of a page tagged bf16 must hold finite K and V, and every in-context page of
    another format keeps poison in the bf16 pools."""
    from workloads import make_workload
    from workloads.configs import attach_mixed_pools, TAG_BF16
    wl = make_workload("mixed_precision", "small", device="cpu")
    rng = np.random.Generator(np.random.PCG64(2024))
    tags = rng.choice([1, 2, 3], size=wl.num_pages, p=[0.4, 0.3, 0.3]).astype(np.uint8)
    attach_mixed_pools(wl, tags, seed=5)
    bt, ctx, b = wl.block_tables.numpy(), wl.context_lens.numpy(), wl.page_size
    k, v = wl.k_pool.float(), wl.v_pool.float()
    n_bf16 = 0
    for r in range(wl.B):
        for t in range(0, int(ctx[r]), b):
            pg, m = int(bt[r, t // b]), min(b, int(ctx[r]) - t)
            if tags[pg] == TAG_BF16:
                n_bf16 += 1
                assert torch.isfinite(k[pg, :, :m]).all() and torch.isfinite(v[pg, :, :, :m]).all()
            else:
                assert torch.isnan(k[pg]).all()
    assert n_bf16 > 0
