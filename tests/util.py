"""Small helpers shared by the tests: tensor <-> numpy conversion and fixture parsing."""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f64(t):
    """Exact float64 copy of a float32/bf16 tensor (or pass numpy through)."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def npy(t):
    """numpy copy of a tensor keeping its dtype (bf16 -> float32, exact)."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            t = t.float()
        return t.numpy().copy()
    return np.array(t)


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def oracle_state(wl):
    """Mutable boundary state of a workload as numpy arrays (K/V upcast exactly to float64)."""
    return dict(
        k_pool=f64(wl.k_pool), v_pool=f64(wl.v_pool),
        block_tables=npy(wl.block_tables).astype(np.int64),
        n_pages=npy(wl.n_pages).astype(np.int64),
        context_lens=npy(wl.context_lens).astype(np.int64),
        refcount=npy(wl.refcount).astype(np.int64),
        free_stack=npy(wl.free_stack).astype(np.int64),
        free_top=npy(wl.free_top).astype(np.int64),
    )
