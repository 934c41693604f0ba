"""Helpers for the GPU parity tests (HIP library through the C ABI vs the CPU oracle)."""
import sys

import numpy as np
import torch

from workloads import make_workload

TOL = {"f32": 2e-4, "bf16": 2e-2}
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


MIXED_POOLS = ("k8", "v8", "k_scale", "v_scale", "page_tag", "k4", "v4", "k4_scale", "v4_scale")


def workload_on_gpu(cfg, scale, page_size=16, int4_frac=0.0):
    """Small workloads are drawn on the CPU and copied (identical values on both sides);
    full-size ones are drawn directly on the GPU."""
    say(f"[workload] {cfg} scale={scale} page_size={page_size} int4_frac={int4_frac}")
    if scale == "small":
        return make_workload(cfg, "small", device="cpu", page_size=page_size,
                             int4_frac=int4_frac).to(DEV)
    return make_workload(cfg, "full", device=DEV, page_size=page_size, int4_frac=int4_frac)


def mixed_np(sub_or_wl):
    """The mixed-precision pools of a workload (or of gather_pages_to_host's dict) as numpy."""
    from util import npy
    g = (lambda n: sub_or_wl[n]) if isinstance(sub_or_wl, dict) else (lambda n: getattr(sub_or_wl, n))
    return {n: npy(g(n)) for n in MIXED_POOLS}


def maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(d)) if d.size else 0.0, bool(np.isnan(d).any())


def sample_requests(wl, n, seed=7):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(wl.B, size=min(n, wl.B), replace=False).tolist())


def gather_pages_to_host(wl, requests):
    """Copy only the pages the listed requests reference (keeps full-size checks cheap)."""
    bt = wl.block_tables[requests].cpu().numpy()
    pages = np.unique(bt[bt >= 0])
    idx = torch.as_tensor(pages, device=wl.k_pool.device, dtype=torch.long)
    remap = np.full(wl.num_pages, -1, dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    sub = dict(k_pool=wl.k_pool.index_select(0, idx).cpu(), v_pool=wl.v_pool.index_select(0, idx).cpu())
    if wl.mixed:
        for name in MIXED_POOLS:
            sub[name] = getattr(wl, name).index_select(0, idx).cpu()
    bt_full = wl.block_tables.cpu().numpy()
    bt_sub = np.full((len(requests), bt_full.shape[1]), -1, dtype=np.int64)
    for i, r in enumerate(requests):
        row = bt_full[r]
        bt_sub[i] = np.where(row >= 0, remap[np.maximum(row, 0)], -1)
    return sub, bt_sub
