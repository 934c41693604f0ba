"""GPU parity: gp_paged_decode_attn (HIP, through the C ABI) vs the float64 oracle."""
import numpy as np
import pytest
import torch

import paged_kv_cache_472_amd as gp
from oracle import attention as oatt
from gpu_common import (DEV, check_decode, decode_reference, gather_pages_to_host, maxabs,
                        mixed_np, sample_requests, say, workload_on_gpu)
from util import f64, npy

pytestmark = pytest.mark.gpu


def _run_gpu(wl, q=None, bt=None, ctx=None, max_context=None):
    cache = gp.KVCache.from_workload(wl)
    out, lse = gp.gp_paged_decode_attn(
        wl.q if q is None else q, cache, wl.block_tables if bt is None else bt,
        wl.context_lens if ctx is None else ctx,
        wl.max_context if max_context is None else max_context, wl.sm_scale)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("cfg,page_size", [("tiny", 16), ("qwen3_8b", 16), ("long_reasoning_d64", 16), ("long_reasoning_d128", 16), ("prefix_shared", 16),
                                            ("mixed_precision", 16), ("tiny", 32), ("long_reasoning_d64", 32), ("prefix_shared", 32), ("mixed_precision", 32),
                                            ("qwen3_8b", 64)])
def test_decode_small_elementwise(cfg, page_size):
    wl = workload_on_gpu(cfg, "small", page_size)
    out, lse = _run_gpu(wl)
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(wl.context_lens), wl.page_size, wl.sm_scale,
                           mixed_np(wl) if wl.mixed else None)
    check_decode(out, lse, ref, wl.dtype, f"decode small {cfg} b={page_size}")


@pytest.mark.parametrize("cfg", ["qwen3_8b", "long_reasoning_d64", "long_reasoning_d128", "prefix_shared", "mixed_precision"])
def test_decode_full_size_sampled(cfg):
    wl = workload_on_gpu(cfg, "full")
    out, lse = _run_gpu(wl)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    reqs = sample_requests(wl, 3)
    sub, bt = gather_pages_to_host(wl, reqs)
    ref = decode_reference(f64(wl.q[reqs]), f64(sub["k_pool"]), f64(sub["v_pool"]), bt,
                           npy(wl.context_lens[reqs]), wl.page_size, wl.sm_scale,
                           mixed_np(sub) if wl.mixed else None)
    check_decode(out[reqs], lse[reqs], ref, wl.dtype, f"decode full {cfg} requests={reqs}")


def test_decode_deterministic_and_grow_bit_identical():
    wl = workload_on_gpu("qwen3_8b", "small")
    o1, l1 = _run_gpu(wl)
    o2, l2 = _run_gpu(wl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # append a free page to every block table without changing the context: output unchanged
    bt = wl.block_tables.clone()
    top = int(wl.free_top.item())
    for r in range(wl.B):
        bt[r, int(wl.n_pages[r])] = int(wl.free_stack[top - 1 - r])
    o3, l3 = _run_gpu(wl, bt=bt)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_decode_edge_cases():
    wl = workload_on_gpu("qwen3_8b", "small")
    ctx = wl.context_lens.clone()
    # empty, one token, exactly one page, a page plus one token; plus a huge max_context bound
    ctx[0], ctx[1], ctx[2] = 0, 1, 16
    out, lse = _run_gpu(wl, ctx=ctx, max_context=wl.max_pages * wl.page_size)
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(ctx), wl.page_size, wl.sm_scale)
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    check_decode(out, lse, ref, "bf16", "decode edge")
    # invalid block-table entries are skipped, never dereferenced
    bt = wl.block_tables.clone()
    bt[1, 0] = -5
    bt[2, 0] = wl.num_pages + 100
    out2, _ = _run_gpu(wl, bt=bt, ctx=ctx)
    assert torch.isfinite(out2.float()).all()
    # a single request, and batch 0
    o1, l1 = gp.gp_paged_decode_attn(wl.q[:1].contiguous(), gp.KVCache.from_workload(wl),
                                    wl.block_tables[:1].contiguous(), wl.context_lens[:1].contiguous(),
                                    wl.max_context, wl.sm_scale)
    torch.cuda.synchronize()
    # a batch of one: other split ranges, against the oracle on its own
    ref1 = decode_reference(f64(wl.q[:1]), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables[:1]),
                            npy(wl.context_lens[:1]), wl.page_size, wl.sm_scale)
    check_decode(o1, l1, ref1, "bf16", "decode single request")


def test_decode_lse_and_split_count_independence():
    """The same request decoded with a different split plan (other batch size) agrees."""
    wl = workload_on_gpu("long_reasoning_d128", "small")
    out, lse = _run_gpu(wl)
    for r in range(wl.B):
        o1, l1 = gp.gp_paged_decode_attn(wl.q[r:r + 1].contiguous(), gp.KVCache.from_workload(wl),
                                         wl.block_tables[r:r + 1].contiguous(),
                                         wl.context_lens[r:r + 1].contiguous(), wl.max_pages * wl.page_size,
                                         wl.sm_scale)
        torch.cuda.synchronize()
        e, _ = maxabs(f64(o1[0]), f64(out[r]))
        el, _ = maxabs(l1[0].cpu().numpy(), lse[r].cpu().numpy())
        assert e <= 1e-2 and el <= 2e-4, (r, e, el)


@pytest.mark.parametrize("max_wg", [1, 5, 37, 224])
def test_decode_capped_grids_match_oracle(max_wg):
    """Grids capped to a few workgroups (ranges long against the batch) against the oracle."""
    wl = workload_on_gpu("long_reasoning_d128", "small")
    out, lse = gp.gp_paged_decode_attn_ex(wl.q, gp.KVCache.from_workload(wl), wl.block_tables,
                                          wl.context_lens, wl.max_context, wl.sm_scale,
                                          max_workgroups=max_wg)
    torch.cuda.synchronize()
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(wl.context_lens), wl.page_size, wl.sm_scale)
    check_decode(out, lse, ref, wl.dtype, f"decode capped {max_wg}")


@pytest.mark.parametrize("cfg", ["tiny", "qwen3_8b", "long_reasoning_d128"])
def test_decode_ring_depths_give_same_bits(cfg):
    """A capped call decodes bf16 / fp32 caches with one tile in flight per wave (an uncapped one
    with two, except over eight-head workgroups of 128-dimensional heads, which also keep one);
    both against the oracle. With 8 KV heads the uncapped kernel holds one workgroup per compute
    unit, so a cap of one workgroup per compute unit keeps the same split of the batch: the same
    tiles in the same order, hence the same bits."""
    wl = workload_on_gpu(cfg, "small")
    cache = gp.KVCache.from_workload(wl)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    o2, l2 = gp.gp_paged_decode_attn_ex(wl.q, cache, wl.block_tables, wl.context_lens,
                                        wl.max_context, wl.sm_scale)
    o1, l1 = gp.gp_paged_decode_attn_ex(wl.q, cache, wl.block_tables, wl.context_lens,
                                        wl.max_context, wl.sm_scale, max_workgroups=cus)
    torch.cuda.synchronize()
    ref = decode_reference(f64(wl.q), f64(wl.k_pool), f64(wl.v_pool), npy(wl.block_tables),
                           npy(wl.context_lens), wl.page_size, wl.sm_scale)
    for depth, (o, l) in ((1, (o1, l1)), (2, (o2, l2))):
        check_decode(o, l, ref, wl.dtype, f"ring depth {depth} {cfg}")
    say(f"[ring depths {cfg}] H_kv={wl.H_kv} equal out={torch.equal(o1, o2)} lse={torch.equal(l1, l2)}")
    if wl.H_kv == 8:
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_decode_graph_replays():
    """A captured decode (stream-K launch and merge) replays with the eager bits, with eager
    calls between the replays."""
    wl = workload_on_gpu("qwen3_8b", "small")
    cache = gp.KVCache.from_workload(wl)
    need = gp.gp_paged_decode_attn_workspace_size(wl.B, wl.H_q, wl.H_kv, wl.q.shape[2],
                                                  wl.page_size, wl.max_context)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(wl.q)
    lse = torch.empty((wl.B, wl.H_q), dtype=torch.float32, device=DEV)
    o_ref, l_ref = gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens,
                                           wl.max_context, wl.sm_scale, workspace=ws)
    o_ref, l_ref = o_ref.clone(), l_ref.clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm the library on the side stream before capturing
        gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens, wl.max_context,
                                wl.sm_scale, out=out, lse=lse, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens, wl.max_context,
                                wl.sm_scale, out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[decode graph] replay {rep}: bit-identical="
            f"{torch.equal(out, o_ref) and torch.equal(lse, l_ref)}")
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
        # eager work between replays
        o2, _ = gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens,
                                        wl.max_context, wl.sm_scale)
        torch.cuda.synchronize()
        assert torch.equal(o2, o_ref)
