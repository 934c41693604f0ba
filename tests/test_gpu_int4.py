"""GPU parity for INT4 pages (PASK App. B.5): the page quantiser bit for bit against the
oracle's quantiser, and decode attention over caches mixing released, fp8, bf16 and INT4 pages
against the float64 oracle (two decode passes with their own stream-K widths, under grid caps)."""
import numpy as np
import pytest
import torch

import paged_kv_cache_472_amd as gp
from oracle import attention as oatt
from oracle import int4 as oi4
from gpu_common import (DEV, check_decode, decode_reference, gather_pages_to_host, mixed_np,
                        sample_requests, say, workload_on_gpu)
from util import f64, npy
from workloads.configs import make_decode_case

pytestmark = pytest.mark.gpu

TAG_FP8, TAG_BF16, TAG_INT4 = 1, 2, 3
K_SENTINEL, V_SENTINEL, S_SENTINEL = 0x5A, 0xA5, 0x7BCD


def _attach_mixed_pools(k, v, b, tags):
    """Mixed-cache pools beside bf16 K/V pools: fp8 pools (unused here) and INT4 pools holding
    sentinels that every conversion must overwrite."""
    P, H, _, D = k.shape
    return gp.KVCache(
        k, v, b,
        k8=torch.zeros((P, H, b, D), dtype=torch.uint8, device=DEV),
        v8=torch.zeros((P, H, D, b), dtype=torch.uint8, device=DEV),
        k_scale=torch.ones((P, H, b), dtype=torch.float32, device=DEV),
        v_scale=torch.ones((P, H, b), dtype=torch.float32, device=DEV),
        page_tag=torch.as_tensor(tags, dtype=torch.uint8, device=DEV),
        k4=torch.full((P, H, b, D // 2), K_SENTINEL, dtype=torch.uint8, device=DEV),
        v4=torch.full((P, H, b // 4, D, 2), V_SENTINEL, dtype=torch.uint8, device=DEV),
        k4_scale=torch.full((P, H, b), S_SENTINEL, dtype=torch.int16, device=DEV).view(torch.float16),
        v4_scale=torch.full((P, H, b), S_SENTINEL, dtype=torch.int16, device=DEV).view(torch.float16))


def _oracle_page(k_page, v_page):
    """Oracle INT4 encoding of one page given as float64 [H, b, D] keys and [H, D, b] values."""
    k4, v4, ks, vs = oi4.quantize_page_kv(k_page, v_page)
    return k4, v4, ks, vs


def _half_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("D,b,H", [(128, 16, 8), (64, 32, 4), (128, 256, 2), (64, 16, 12)])
def test_quantize_pages_bit_exact(D, b, H):
    P = 12
    gen = torch.Generator(device="cpu").manual_seed(D * 1000 + b + H)
    k = torch.randn((P, H, b, D), generator=gen) * torch.exp2(torch.randint(-12, 6, (P, H, b, 1), generator=gen).float())
    v = torch.randn((P, H, D, b), generator=gen) * torch.exp2(torch.randint(-12, 6, (P, H, 1, b), generator=gen).float())
    # special rows: a zero row, a row below the 2^-24 floor, a row of rounding ties, a subnormal
    # scale that clips, and a heavy outlier
    k[0, 0, 0] = 0.0
    v[0, 0, :, 0] = 0.0
    k[0, 0, 1] = 1e-12
    v[0, 0, :, 1] = -1e-12
    tie = torch.tensor([7.0, 2.5, -0.5, 1.5, -3.5, 0.5, 6.5, -6.5] * (D // 8))
    k[1, 0, 2] = tie
    v[1, 0, :, 2] = tie
    k[1, 0, 3] = 0.0
    k[1, 0, 3, :3] = torch.tensor([39 * 2.0 ** -26, -4.5 * 2.0 ** -24, 1.5 * 2.0 ** -24])
    k[2, 0, 4, 5] = 3e4
    k, v = k.to(torch.bfloat16), v.to(torch.bfloat16)
    tags = np.full(P, TAG_BF16, dtype=np.uint8)
    tags[5] = TAG_FP8                           # listed but not bf16: must stay untouched
    cache = _attach_mixed_pools(k.to(DEV), v.to(DEV), b, tags)
    ids = [0, 1, 2, 5, 7, 9, 9, -1, P + 3, 11]  # a repeat and two ids out of range
    say(f"[quantize D={D} b={b} H={H}] ids={ids}")
    gp.gp_quantize_pages_int4(cache, torch.as_tensor(ids, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    got_tags = cache.page_tag.cpu().numpy()
    k4, v4 = cache.k4.cpu().numpy(), cache.v4.cpu().numpy()
    ks = cache.k4_scale.cpu().view(torch.int16).numpy().view(np.uint16)
    vs = cache.v4_scale.cpu().view(torch.int16).numpy().view(np.uint16)
    converted = {0, 1, 2, 7, 9, 11}
    for pg in range(P):
        if pg in converted:
            assert got_tags[pg] == TAG_INT4
            ek4, ev4, eks, evs = _oracle_page(f64(k[pg]), f64(v[pg]))
            assert np.array_equal(k4[pg], ek4), f"k codes of page {pg}"
            assert np.array_equal(v4[pg], ev4), f"v codes of page {pg}"
            assert np.array_equal(ks[pg], _half_bits(eks)), f"k scales of page {pg}"
            assert np.array_equal(vs[pg], _half_bits(evs)), f"v scales of page {pg}"
        else:
            assert got_tags[pg] == tags[pg]
            assert (k4[pg] == K_SENTINEL).all() and (v4[pg] == V_SENTINEL).all()
            assert (ks[pg] == S_SENTINEL).all() and (vs[pg] == S_SENTINEL).all()
    # the special rows landed where the oracle says (sanity of the fixture itself)
    assert ks[0, 0, 0] == 0x3C00 and ks[0, 0, 1] == 0x0001


def _run_decode(wl, cache=None):
    cache = gp.KVCache.from_workload(wl) if cache is None else cache
    out, lse = gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens,
                                       wl.max_context, wl.sm_scale)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("page_size,int4_frac", [(16, 0.5), (32, 0.5), (16, 1.0)])
def test_decode_int4_small_elementwise(page_size, int4_frac):
    wl = workload_on_gpu("mixed_precision", "small", page_size, int4_frac=int4_frac)
    tags = npy(wl.page_tag)
    used = np.unique(npy(wl.block_tables)[npy(wl.block_tables) >= 0])
    assert set(np.unique(tags[used])) >= {TAG_INT4, TAG_BF16 if int4_frac < 1 else TAG_INT4}
    out, lse = _run_decode(wl)
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(wl.context_lens), wl.page_size, wl.sm_scale, mixed_np(wl))
    check_decode(out, lse, ref, "bf16", f"decode int4 small b={page_size} frac={int4_frac}")


def test_decode_int4_full_size_sampled():
    wl = workload_on_gpu("mixed_precision", "full", int4_frac=0.5)
    out, lse = _run_decode(wl)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    reqs = sample_requests(wl, 3)
    sub, bt = gather_pages_to_host(wl, reqs)
    ref = decode_reference(f64(wl.q[reqs]), f64(sub["k_pool"]), f64(sub["v_pool"]), bt,
                           npy(wl.context_lens[reqs]), wl.page_size, wl.sm_scale, mixed_np(sub))
    check_decode(out[reqs], lse[reqs], ref, "bf16", f"decode int4 full requests={reqs}")


@pytest.mark.parametrize("D,b,G", [(64, 16, 4), (128, 32, 1), (64, 64, 16), (128, 256, 4)])
def test_quantize_then_decode(D, b, G):
    """Demote every other used page on the GPU, decode there; the oracle demotes the same pages
    with its own quantiser and decodes."""
    H_kv = 2
    rng = np.random.default_rng(D + b + G)
    lens = rng.integers(0, 900, size=6)
    lens[0] = 0
    wl = make_decode_case(6, G * H_kv, H_kv, D, b, lens, dtype="bf16", seed=D * b + G).to(DEV)
    bt = npy(wl.block_tables)
    used = np.unique(bt[bt >= 0])
    demote = used[::2]
    tags = np.full(wl.num_pages, TAG_BF16, dtype=np.uint8)
    cache = _attach_mixed_pools(wl.k_pool, wl.v_pool, b, tags)
    say(f"[quantize+decode D={D} b={b} G={G}] demoted {len(demote)} of {len(used)} pages")
    gp.gp_quantize_pages_int4(cache, torch.as_tensor(demote, dtype=torch.int32, device=DEV))
    out, lse = _run_decode(wl, cache)
    # oracle side: its own encoding of the same pages (dead rows hold NaN; zero them first,
    # they are never read)
    kp, vp = f64(wl.k_pool), f64(wl.v_pool)
    k4 = np.zeros(cache.k4.shape, dtype=np.uint8)
    v4 = np.zeros(cache.v4.shape, dtype=np.uint8)
    ks = np.ones(cache.k4_scale.shape)
    vs = np.ones(cache.v4_scale.shape)
    for pg in demote:
        k4[pg], v4[pg], ks[pg], vs[pg] = _oracle_page(np.nan_to_num(kp[pg], nan=0.0),
                                                      np.nan_to_num(vp[pg], nan=0.0))
    otags = tags.copy()
    otags[demote] = TAG_INT4
    z8 = np.zeros(1, dtype=np.uint8)
    ref = decode_reference(f64(wl.q), kp, vp, bt, npy(wl.context_lens), b, wl.sm_scale,
                           dict(page_tag=otags, k8=z8, v8=z8, k_scale=z8, v_scale=z8, k4=k4, v4=v4,
                                k4_scale=ks, v4_scale=vs))
    assert np.array_equal(cache.page_tag.cpu().numpy(), otags)
    check_decode(out, lse, ref, "bf16", f"quantize+decode D={D} b={b} G={G}")
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))


@pytest.mark.parametrize("max_wg,H_kv", [(1, 8), (3, 4), (37, 8), (100000, 8), (100000, 2)])
def test_mixed_two_passes_capped_grid(max_wg, H_kv):
    """A mixed cache (released / fp8 / bf16 / INT4 pages) decodes in two passes whose stream-K
    widths differ (the INT4 pass uses four-head workgroups); under any grid cap the merged
    result must match the oracle."""
    from workloads.configs import attach_mixed_pools
    lens = [0, 5, 700, 16, 3000, 1, 0, 257, 1200, 64, 4000]
    wl = make_decode_case(len(lens), 4 * H_kv, H_kv, 128, 16, lens, seed=max_wg % 89 + H_kv).to(DEV)
    tags = np.random.default_rng(max_wg + H_kv).choice([0, 1, 2, 3], size=wl.num_pages,
                                                       p=[0.15, 0.25, 0.3, 0.3]).astype(np.uint8)
    attach_mixed_pools(wl, tags, seed=H_kv)
    say(f"[two passes cap={max_wg} H_kv={H_kv}] tags used={np.bincount(tags, minlength=4).tolist()}")
    out, lse = gp.gp_paged_decode_attn_ex(wl.q, gp.KVCache.from_workload(wl), wl.block_tables,
                                          wl.context_lens, wl.max_context, wl.sm_scale,
                                          max_workgroups=max_wg)
    torch.cuda.synchronize()
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(wl.context_lens), 16, wl.sm_scale, mixed_np(wl))
    check_decode(out, lse, ref, "bf16", f"two passes cap={max_wg} H_kv={H_kv}")
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
