"""Pins for the decode-attention oracle (PASK Sec. 3.1 and App. B.5) and the fp8 decoder."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as oatt
from oracle.fp8 import e4m3_decode
from workloads import make_workload
from util import f64, golden_lines, npy


# ----------------------------------------------------------------------------- fp8
def test_e4m3_all_codes_match_library():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], lib[~nan])
    assert nan.sum() == 2


def test_e4m3_golden():
    for code, val in golden_lines("e4m3_codes.txt"):
        got = e4m3_decode(np.array([int(code, 16)], dtype=np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


# ----------------------------------------------------------------------------- attention
def test_decode_golden_two_tokens():
    rows = {r[0]: [float(x) for x in r[1:]] for r in golden_lines("decode_tiny.txt")}
    q = np.array([rows["q"]])
    k = np.array([rows["k1"], rows["k2"]])
    v = np.array([rows["v1"], rows["v2"]])
    o, lse = oatt.attend(q, k, v, 1.0)
    assert np.allclose(o[0], rows["o"], rtol=0, atol=1e-12)
    assert abs(lse[0] - rows["lse"][0]) < 1e-12


def test_decode_gqa_golden():
    """Hand-worked GQA decode (tests/golden/decode_gqa.txt): query head g reads KV head g // G."""
    rows = {r[0]: np.array([float(x) for x in r[1:]]) for r in golden_lines("decode_gqa.txt")}
    b, d = 16, 2
    q = rows["q"].reshape(1, 4, d)
    k_pool = np.full((1, 2, b, d), np.nan)
    v_pool = np.full((1, 2, d, b), np.nan)
    for h in range(2):
        k_pool[0, h, :2] = rows[f"k_h{h}"].reshape(2, d)
        v_pool[0, h, :, :2] = rows[f"v_h{h}"].reshape(2, d).T
    out, lse = oatt.paged_decode_attn(q, k_pool, v_pool, np.array([[0]]), np.array([2]), b, 1.0)
    assert np.allclose(out[0], rows["o"].reshape(4, d), rtol=0, atol=1e-12)
    assert np.allclose(lse[0], rows["lse"], rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 32))
    k = rng.standard_normal((300, 32)) * 3
    o, lse = oatt.attend(q, k, np.ones((300, 32)), 1 / math.sqrt(32))
    assert np.allclose(o, 1.0, atol=1e-12)
    z = q @ k.T / math.sqrt(32)
    assert np.allclose(np.exp(z - lse[:, None]).sum(axis=1), 1.0, atol=1e-12)


def test_empty_context_gives_zero_and_neg_inf():
    o, lse = oatt.attend(np.ones((2, 8)), np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def _contiguous_copy(wl):
    """Same tokens, block tables rewritten to identity order 0..P-1 per request."""
    b = wl.page_size
    bt = npy(wl.block_tables)
    kp, vp = f64(wl.k_pool), f64(wl.v_pool)
    k2, v2, bt2 = [], [], np.full_like(bt, -1)
    nxt = 0
    for r in range(wl.B):
        P = int(wl.n_pages[r])
        for j in range(P):
            k2.append(kp[bt[r, j]])
            v2.append(vp[bt[r, j]])
            bt2[r, j] = nxt
            nxt += 1
    return np.stack(k2), np.stack(v2), bt2


@pytest.mark.parametrize("cfg", ["tiny", "qwen3_8b", "prefix_shared"])
def test_permutation_invariance(cfg):
    wl = make_workload(cfg, "small")
    q = f64(wl.q)
    ctx = npy(wl.context_lens)
    o1, l1 = oatt.paged_decode_attn(q, f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                                    ctx, wl.page_size, wl.sm_scale)
    k2, v2, bt2 = _contiguous_copy(wl)
    o2, l2 = oatt.paged_decode_attn(q, k2, v2, bt2, ctx, wl.page_size, wl.sm_scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isfinite(o1).all()


@pytest.mark.parametrize("cfg", ["tiny", "long_reasoning_d128"])
def test_matches_torch_sdpa_float64(cfg):
    wl = make_workload(cfg, "small")
    q = f64(wl.q)
    o, lse = oatt.paged_decode_attn(q, f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                                    npy(wl.context_lens), wl.page_size, wl.sm_scale)
    for r in range(wl.B):
        k, v, _ = oatt.gather_request_kv(r, f64(wl.k_pool), f64(wl.v_pool),
                                         npy(wl.block_tables), npy(wl.context_lens), wl.page_size)
        for h in range(wl.H_kv):
            qs = torch.from_numpy(q[r, h * wl.G:(h + 1) * wl.G])[None, :, None, :]
            ks = torch.from_numpy(k[h])[None, None].expand(1, wl.G, -1, -1)
            vs = torch.from_numpy(v[h])[None, None].expand(1, wl.G, -1, -1)
            ref = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs)[0, :, 0].numpy()
            assert np.allclose(o[r, h * wl.G:(h + 1) * wl.G], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cfg", ["tiny", "long_reasoning_d128", "prefix_shared"])
def test_gqa_mapping_matches_repeated_kv_sdpa(cfg):
    """GQA pinned apart from the oracle's head slicing: K/V gathered here straight from the pools
    (K [page, head, slot, d], V [page, head, d, slot]), repeated G times along the head axis with
    torch.repeat_interleave (query head g sees KV head g // G), and attended by torch SDPA for all
    query heads at once in float64."""
    wl = make_workload(cfg, "small")
    q, kp, vp = f64(wl.q), f64(wl.k_pool), f64(wl.v_pool)
    bt, ctx, b = npy(wl.block_tables), npy(wl.context_lens), wl.page_size
    o, _ = oatt.paged_decode_attn(q, kp, vp, bt, ctx, b, wl.sm_scale)
    for r in range(wl.B):
        n = int(ctx[r])
        if n == 0:
            continue
        t = np.arange(n)
        pg, sl = bt[r, t // b], t % b
        k = kp[pg, :, sl, :].transpose(1, 0, 2)        # [H_kv, n, d]
        v = vp[pg, :, :, sl].transpose(1, 0, 2)        # [H_kv, n, d]
        kr = torch.from_numpy(np.ascontiguousarray(k)).repeat_interleave(wl.G, dim=0)
        vr = torch.from_numpy(np.ascontiguousarray(v)).repeat_interleave(wl.G, dim=0)
        qs = torch.from_numpy(q[r])[:, None, :]        # [H_q, 1, d]
        ref = torch.nn.functional.scaled_dot_product_attention(qs, kr, vr, scale=wl.sm_scale)
        assert np.allclose(o[r], ref[:, 0].numpy(), rtol=0, atol=1e-12)


def test_split_merge_equals_single_pass():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 16))
    k = rng.standard_normal((257, 16)) * 2
    v = rng.standard_normal((257, 16))
    o, lse = oatt.attend(q, k, v, 0.25)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 257), size=trial + 1, replace=False))
        bounds = [0, *cuts.tolist(), 257]
        parts = [oatt.split_partial(q, k[a:b], v[a:b], 0.25) for a, b in zip(bounds, bounds[1:])]
        o2, lse2 = oatt.merge_splits(parts)
        assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)


def _mixed(wl):
    return dict(page_tag=npy(wl.page_tag), k8=npy(wl.k8), v8=npy(wl.v8),
                k_scale=npy(wl.k_scale), v_scale=npy(wl.v_scale), k4=npy(wl.k4), v4=npy(wl.v4),
                k4_scale=npy(wl.k4_scale), v4_scale=npy(wl.v4_scale))


def _nibble(byte_array, high):
    """Signed nibble by arithmetic shifts of int8 (an independent route to the code)."""
    b = np.asarray(byte_array, dtype=np.uint8)
    if not high:
        b = (b << 4).astype(np.uint8)
    return (b.view(np.int8) >> 4).astype(np.float64)


@pytest.mark.parametrize("int4_frac", [0.0, 0.5])
def test_released_page_equals_deleting_its_tokens(int4_frac):
    wl = make_workload("mixed_precision", "small", int4_frac=int4_frac)
    args = (f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables), npy(wl.context_lens),
            wl.page_size)
    mixed = _mixed(wl)
    out, lse = oatt.paged_decode_attn(f64(wl.q), *args[:4], wl.page_size, wl.sm_scale, **mixed)
    assert np.isfinite(out).all()
    tags = npy(wl.page_tag)
    b = wl.page_size
    for r in range(wl.B):
        n = int(wl.context_lens[r])
        # tokens of pages that are not released, decoded by hand from the three tag kinds
        ks, vs = [], []
        for j in range(n):
            pg, off = int(wl.block_tables[r, j // b]), j % b
            if tags[pg] == 0:
                continue
            if tags[pg] == 2:
                ks.append(f64(wl.k_pool)[pg, :, off, :])
                vs.append(f64(wl.v_pool)[pg, :, :, off])
            elif tags[pg] == 3:
                kb = npy(wl.k4)[pg, :, off, :]                       # [H, d/2]
                kc = np.stack([_nibble(kb, False), _nibble(kb, True)], -1).reshape(wl.H_kv, wl.d)
                slot = (np.arange(wl.d) % 16) * (wl.d // 16) + np.arange(wl.d) // 16
                vb = npy(wl.v4)[pg, :, off // 4][:, slot, (off % 4) // 2]      # [H, d]
                vc = _nibble(vb, off % 2 == 1)
                ks.append(kc * npy(wl.k4_scale)[pg, :, off, None].astype(np.float64))
                vs.append(vc * npy(wl.v4_scale)[pg, :, off, None].astype(np.float64))
            else:
                ks.append(e4m3_decode(npy(wl.k8)[pg, :, off, :]) * npy(wl.k_scale)[pg, :, off, None])
                vs.append(e4m3_decode(npy(wl.v8)[pg, :, :, off]) * npy(wl.v_scale)[pg, :, off, None])
        if int4_frac:
            assert (tags[npy(wl.block_tables)[r, :(n + wl.page_size - 1) // wl.page_size]] == 3).any()
        K, V = np.stack(ks, 1), np.stack(vs, 1)
        for h in range(wl.H_kv):
            o, l_ = oatt.attend(f64(wl.q)[r, h * wl.G:(h + 1) * wl.G], K[h], V[h], wl.sm_scale)
            assert np.allclose(out[r, h * wl.G:(h + 1) * wl.G], o, rtol=0, atol=1e-12)
            assert np.allclose(lse[r, h * wl.G:(h + 1) * wl.G], l_, atol=1e-12)


def test_int4_page_equals_float_page_of_its_values():
    """Dequantised through the oracle's own unpacking, an INT4 page must give the same output
    as a float page holding code * scale; the values come from arithmetic shifts here."""
    wl = make_workload("mixed_precision", "small", int4_frac=1.0)
    tags = npy(wl.page_tag)
    assert (tags == 3).any()
    kp, vp = f64(wl.k_pool), f64(wl.v_pool)
    for pg in np.nonzero(tags == 3)[0]:
        kb = npy(wl.k4)[pg]                                            # [H, b, d/2]
        kc = np.stack([_nibble(kb, False), _nibble(kb, True)], -1).reshape(kp.shape[1:])
        slot = (np.arange(wl.d) % 16) * (wl.d // 16) + np.arange(wl.d) // 16
        vb = npy(wl.v4)[pg][:, :, slot, :]                             # [H, b/4, d, 2]
        vc = np.stack([_nibble(vb, False), _nibble(vb, True)], -1)     # [H, Q, d, k, 2]
        vc = vc.transpose(0, 2, 1, 3, 4).reshape(vp.shape[1:])         # [H, d, b]
        kp[pg] = kc * npy(wl.k4_scale)[pg][..., None].astype(np.float64)
        vp[pg] = vc * npy(wl.v4_scale)[pg][:, None, :].astype(np.float64)
    float_tags = np.where(tags == 3, 2, tags).astype(np.uint8)
    mixed = _mixed(wl)
    o1, l1 = oatt.paged_decode_attn(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool),
                                    npy(wl.block_tables), npy(wl.context_lens), wl.page_size,
                                    wl.sm_scale, **mixed)
    mixed["page_tag"] = float_tags
    o2, l2 = oatt.paged_decode_attn(f64(wl.q), kp, vp, npy(wl.block_tables),
                                    npy(wl.context_lens), wl.page_size, wl.sm_scale, **mixed)
    assert np.isfinite(o1).all()
    assert np.allclose(o1, o2, rtol=0, atol=1e-12) and np.allclose(l1, l2, rtol=0, atol=1e-12)


def test_all_pages_released_gives_zero():
    wl = make_workload("mixed_precision", "small")
    tags = np.zeros_like(npy(wl.page_tag))
    out, lse = oatt.paged_decode_attn(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool),
                                      npy(wl.block_tables), npy(wl.context_lens), wl.page_size,
                                      wl.sm_scale, page_tag=tags, k8=npy(wl.k8), v8=npy(wl.v8),
                                      k_scale=npy(wl.k_scale), v_scale=npy(wl.v_scale))
    assert np.all(out == 0) and np.all(np.isneginf(lse))
