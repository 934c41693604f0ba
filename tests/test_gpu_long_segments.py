"""GPU parity for decode segments longer than one tile list.

A wave lists at most 256 tiles (4096 tokens) of its segment in LDS at a time and walks them;
a longer segment is listed and walked again from where the previous list stopped, carrying the
running softmax state across the seam. With the grid capped to one or two workgroups, requests
of 4097-7001 tokens are decoded as single segments of 257-438 tiles, so every list seam (and a
segment that ends one token after a seam) is crossed, for fp32 and bf16 caches, a mixed cache
of bf16 and fp8 pages, and one that adds INT4 and released pages (PASK Sec. 3.1, App. B.5).
Checked element by element against the float64 oracle: lse at the fp32 bound.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_472_amd as gp
from gpu_common import DEV, check_decode, decode_reference, mixed_np, say
from util import f64, npy
from workloads.configs import attach_mixed_pools, make_decode_case

pytestmark = pytest.mark.gpu

LENS = [6000, 300, 7001, 0, 4097, 4096]


@pytest.mark.parametrize("kind", ["f32", "bf16", "fp8_mixed", "int4_mixed"])
@pytest.mark.parametrize("max_wg", [1, 2])
def test_decode_segments_past_one_tile_list(kind, max_wg):
    dtype = "f32" if kind == "f32" else "bf16"
    wl = make_decode_case(len(LENS), 8, 2, 128, 16, LENS, dtype=dtype, seed=41 + max_wg).to(DEV)
    if kind.endswith("_mixed"):
        rng = np.random.default_rng(7 + max_wg)
        if kind == "fp8_mixed":
            tags = rng.choice([1, 2], size=wl.num_pages).astype(np.uint8)          # fp8 / bf16
        else:
            tags = rng.choice([0, 1, 2, 3], size=wl.num_pages,
                              p=[0.1, 0.3, 0.3, 0.3]).astype(np.uint8)
        attach_mixed_pools(wl, tags, seed=max_wg)
    tiles = [-(-n // 16) for n in LENS]
    say(f"[long segments {kind} cap={max_wg}] tiles per request {tiles} (list of 256)")
    out, lse = gp.gp_paged_decode_attn_ex(wl.q, gp.KVCache.from_workload(wl), wl.block_tables,
                                          wl.context_lens, wl.max_context, wl.sm_scale,
                                          max_workgroups=max_wg)
    torch.cuda.synchronize()
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(wl.context_lens), 16, wl.sm_scale,
                           mixed_np(wl) if wl.mixed else None)
    check_decode(out, lse, ref, dtype, f"long segments {kind} cap={max_wg}")
    assert torch.all(out[3] == 0) and torch.all(torch.isneginf(lse[3]))
