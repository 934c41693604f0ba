"""gp_paged_decode_attn_noalloc (split partials in the library's static device buffer, no
workspace) against gp_paged_decode_attn_ex with a caller workspace, through the C ABI: the same
bits on two calls in a row, the second with a smaller batch and context bound (the buffer then
holds the first call's partials), over a bf16 cache with the fused summary update and a capped
grid, and over a mixed cache (two passes). The first call is also checked against the oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_472_amd as gp
from gpu_common import DEV, check_decode, decode_reference, mixed_np, say
from util import f64, npy
from workloads.configs import attach_mixed_pools, make_decode_case

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _sub(wl, n):
    return (wl.q[:n].contiguous(), wl.block_tables[:n].contiguous(),
            wl.context_lens[:n].contiguous(), int(wl.context_lens[:n].max()))


def _both(wl, q, bt, ctx, max_ctx, cap, with_summaries):
    cache = gp.KVCache.from_workload(wl)
    outs = []
    for entry in (gp.gp_paged_decode_attn_ex, gp.gp_paged_decode_attn_noalloc):
        upd = None
        if with_summaries:
            upd = dict(q_pre=q, slot_ids=wl.slot_ids[:q.shape[0]].contiguous(),
                       fresh=torch.zeros(q.shape[0], dtype=torch.uint8, device=DEV),
                       qstate=wl.qstate.clone(), beta_s=0.9, beta_l=0.999)
        o, l_ = entry(q, cache, bt, ctx, max_ctx, wl.sm_scale, summaries=upd, max_workgroups=cap)
        torch.cuda.synchronize()
        outs.append((o, l_, None if upd is None else upd["qstate"]))
    return outs


@pytest.mark.parametrize("kind", ["bf16", "mixed"])
def test_noalloc_equals_workspace_call_twice(kind):
    lens = [3000, 17, 0, 5000, 640, 2049, 1, 4100]
    wl = make_decode_case(len(lens), 32, 8, 128, 16, lens, seed=77).to(DEV)
    if kind == "mixed":
        tags = np.random.default_rng(5).choice([0, 1, 2, 3], size=wl.num_pages,
                                               p=[0.1, 0.3, 0.3, 0.3]).astype(np.uint8)
        attach_mixed_pools(wl, tags, seed=5)
    wl.qstate.normal_()
    cap = 0 if kind == "mixed" else 100
    for call, n in enumerate((len(lens), 3)):            # the second call is smaller
        q, bt, ctx, max_ctx = _sub(wl, n)
        (o1, l1, s1), (o2, l2, s2) = _both(wl, q, bt, ctx, max_ctx, cap, kind == "bf16")
        same = torch.equal(_bits(o1), _bits(o2)) and torch.equal(_bits(l1), _bits(l2))
        if s1 is not None:
            same = same and torch.equal(_bits(s1), _bits(s2))
        say(f"[noalloc {kind} call {call}] batch {n}, max_context {max_ctx}: bits equal={same}")
        assert same
        if call == 0:
            ref = decode_reference(f64(q), f64(wl.k_pool), f64(wl.v_pool), npy(bt), npy(ctx), 16,
                                   wl.sm_scale, mixed_np(wl) if wl.mixed else None)
            check_decode(o2, l2, ref, "bf16", f"noalloc {kind} vs oracle")
