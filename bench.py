"""Benchmark of the paged-KV hot path on one MI355X.

One step is one pass of the whole path over one batch of the Qwen3-8B-shaped decode layer
(64 requests, contexts uniform in [4096, 16384], 32 query / 8 KV heads, head_dim 128, 16-token
pages, bf16): the dual-timescale summary update of every request, paged decode attention of
every request (split partials plus their merge), and the page-boundary pass of the requests that
sit at a page boundary (scores, working sets, compress-or-grow with compaction). Compaction and
page growth are destructive, so each step first restores the small integer page state (block
tables, lengths, page counts, refcounts, free stack) with one device copy, inside the timed
region; K/V pages are left as the previous step's compaction wrote them (still valid tokens, same
amount of work).

By default (--overlap 1) the step overlaps the boundary pass with decoding, as GrowPage does
(App. E.3). The main stream decodes every request from a copy of the block tables and lengths
taken by the restore, with the summary update of the requests that are not at a boundary fused
into the call and a grid that leaves --reserve-cus compute units free. A second stream meanwhile
updates the boundary requests' summaries, scores them and plans their compress-or-grow
(decisions, page allocation, kept tokens: bookkeeping on the live tables only); the planned K/V
movement runs on the main stream after the decode, with the whole GPU. Every request still sees
update -> decode -> boundary pass in that order. --overlap 0 runs the same rows one after another
on one stream.

Prints one JSON line. `value` is the step's algorithmic HBM bytes divided by the step time;
`roofline` is the main decode call (its two kernels) against the 8 TB/s HBM peak, timed with HIP
events on the stream it is launched on; `cpu_baseline` is the float64 CPU oracle on a bounded
sample of the same workload. `int4_decode` (bf16 workloads, --int4 1) times decode of the same
batch after every used page has been demoted to INT4 pages by the page quantiser (PASK App. B.5):
the quantiser call itself, the decode time per launch and its bytes against the same peak.
`decode_configs` (--decode-configs 1) times one decode call of the whole batch of the tiny,
long-reasoning (both head shapes), prefix-shared and mixed-precision workloads at full size:
median time, bytes on the same model (the prefix-shared batch also with each shared token counted
once), GB/s and the fraction of the 8 TB/s peak.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MIXED_POOLS = ("k8", "v8", "k_scale", "v_scale", "page_tag", "k4", "v4", "k4_scale", "v4_scale")
METRIC = "paged decode attention KV GB/s (% HBM peak) + boundary-pass latency/request"
PMC_FILE = os.path.join(ROOT, "profiles", "decode_qwen3_8b_traffic.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_472_amd", "csrc", "decode.hip")

WORKLOAD_NAMES = {
    "tiny": "tiny decode step (B=2, ctx 200/333, Hq=8, Hkv=2, d=64, fp32)",
    "qwen3_8b": "Qwen3-8B-shaped decode layer (B=64, ctx U[4096,16384], Hq=32, Hkv=8, d=128, b=16, bf16)",
    "long_reasoning_d64": "long-reasoning mix, 8/2 heads d=64 (B=256, lognormal ctx, bf16)",
    "long_reasoning_d128": "long-reasoning mix, 32/8 heads d=128 (B=256, lognormal ctx, bf16)",
    "prefix_shared": "prefix-shared batch (B=128, shared 2048 + U[1024,8192], Hq=40, Hkv=8, d=128, bf16)",
    "mixed_precision": "mixed-precision pages (B=128, ctx U[8192,24576], 30/40/30 release/fp8/bf16)",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle's timed sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--reserve-cus", type=int, default=32,
                    help="with --overlap 1 or 2: compute units the main decode leaves free for the "
                         "boundary pass on the second stream (its workgroup cap; 0: no cap)")
    ap.add_argument("--overlap", type=int, default=1,
                    help="1: the boundary pass runs on a second stream beside the decode (its K/V "
                         "movement after it); 2: the boundary requests are scored first, then the "
                         "decode runs beside their compress-or-grow plan; 0: everything on one "
                         "stream")
    ap.add_argument("--int4", type=int, default=1,
                    help="also time decode with every page of the batch demoted to INT4 "
                         "(PASK App. B.5) by the page quantiser (bf16 workloads)")
    ap.add_argument("--boundary-pass", type=int, default=1,
                    help="also time the boundary pass alone on the long-reasoning, prefix-shared "
                         "and tiny workloads (16- and 256-token pages)")
    ap.add_argument("--decode-configs", type=int, default=1,
                    help="also time one decode call of the whole batch on the tiny, long-reasoning, "
                         "prefix-shared and mixed-precision workloads (GB/s and fraction of peak)")
    ap.add_argument("--copy-probe-gib", type=float, default=1.0,
                    help="size of the plain device copy timed beside the path (HBM reference)")
    return ap.parse_args()


def file_sha(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


class Path:
    """Preallocated buffers and the per-step launch sequence of one workload."""

    def __init__(self, wl, gp, torch, overlap=False, reserve_cus=0):
        self.wl, self.gp, self.torch = wl, gp, torch
        dev = wl.q.device
        i32 = torch.int32
        self.R = wl.req_idx.numel()
        self.overlap = bool(overlap) and self.R > 0
        self.mode = int(overlap) if self.overlap else 0
        # integer page state in one flat buffer so a step can restore it with one copy; with
        # overlap it also holds a second copy of the block tables and lengths that the decode
        # reads, so that the boundary pass may rewrite the live ones while the decode runs
        names = ("block_tables", "n_pages", "context_lens", "refcount", "free_stack", "free_top")
        sizes = [getattr(wl, n).numel() for n in names]
        extra = wl.block_tables.numel() + wl.B
        self.meta = torch.empty(sum(sizes) + extra, dtype=i32, device=dev)
        off = 0
        for n, sz in zip(names, sizes):
            t = getattr(wl, n)
            view = self.meta[off:off + sz].view(t.shape)
            view.copy_(t)
            setattr(wl, n, view)
            off += sz
        self.bt_dec = self.meta[off:off + wl.block_tables.numel()].view(wl.block_tables.shape)
        self.bt_dec.copy_(wl.block_tables)
        off += wl.block_tables.numel()
        self.ctx_dec = self.meta[off:off + wl.B]
        self.ctx_dec.copy_(wl.context_lens)
        self.meta0 = self.meta.clone()
        self.cache = gp.KVCache.from_workload(wl)
        B, H_q, d = wl.q.shape
        H_kv = wl.H_kv
        self.out = torch.empty_like(wl.q)
        self.lse = torch.empty((B, H_q), dtype=torch.float32, device=dev)
        n = gp.gp_paged_decode_attn_workspace_size(B, H_q, H_kv, d, wl.page_size, wl.max_context)
        self.dws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
        self.fresh0 = torch.zeros(B, dtype=torch.uint8, device=dev)
        self.upd = dict(q_pre=wl.q, slot_ids=wl.slot_ids, fresh=self.fresh0, qstate=wl.qstate,
                        beta_s=wl.beta_s, beta_l=wl.beta_l)
        self.max_wg = 0
        if self.R:
            req = wl.req_idx.cpu().tolist()
            ctx = wl.context_lens.cpu().tolist()
            b = wl.page_size
            cm = max(max(0, (math.ceil(ctx[r] / b) - 1) * b) for r in req)
            self.C_max = max(16, -(-cm // 16) * 16)
            R, C = self.R, self.C_max
            self.a_s = torch.empty((R, H_kv, C), dtype=torch.float32, device=dev)
            self.a_l = torch.empty_like(self.a_s)
            self.wsc = torch.empty((R, H_kv, 2), dtype=i32, device=dev)
            self.ncand = torch.empty((R,), dtype=i32, device=dev)
            n = gp.gp_score_and_working_set_workspace_size(R, H_q, H_kv, d, b, C)
            self.sws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
            self.dec = torch.empty((R,), dtype=i32, device=dev)
            self.kept = torch.empty((R, H_kv, C), dtype=i32, device=dev)
            n = gp.gp_compact_or_grow_workspace_size(R, H_kv, wl.max_pages, b, C)
            self.cws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
            self.policies = torch.as_tensor(wl.req_policy, dtype=i32, device=dev)
        if self.overlap:
            self.stream_b = torch.cuda.Stream(device=dev)  # default priority
            self.req_l = wl.req_idx.long()
            # the decode updates the summaries of the other requests; the second stream updates
            # the boundary requests' own before their scores read them
            slot_main = wl.slot_ids.clone()
            slot_main.index_fill_(0, self.req_l, -1)
            self.upd_main = dict(self.upd, slot_ids=slot_main)
            self.slot_b = torch.full_like(wl.slot_ids, -1)
            self.slot_b[self.req_l] = wl.slot_ids[self.req_l]
            cus = torch.cuda.get_device_properties(dev).multi_processor_count
            self.max_wg = max(1, cus - reserve_cus) if reserve_cus > 0 else 0
            self.ev_a = torch.cuda.Event()
            self.ev_b = torch.cuda.Event()

    def build_state(self):
        """Summaries after the past queries (first one initialises the slot)."""
        wl, gp, torch = self.wl, self.gp, self.torch
        ones = torch.ones_like(self.fresh0)
        for t in range(wl.q_hist.shape[0]):
            gp.gp_update_query_summaries(wl.q_hist[t].contiguous(), wl.slot_ids,
                                         ones if t == 0 else self.fresh0, wl.qstate,
                                         wl.beta_s, wl.beta_l)

    def step(self, ev=None):
        wl, gp = self.wl, self.gp
        rec = (lambda k: ev[k] is not None and ev[k].record()) if ev is not None else (lambda k: None)
        rec(0)
        self.meta.copy_(self.meta0)
        rec(1)
        rec(2)
        gp.gp_paged_decode_attn_ex(wl.q, self.cache, wl.block_tables, wl.context_lens,
                                   wl.max_context, wl.sm_scale, summaries=self.upd, out=self.out,
                                   lse=self.lse, workspace=self.dws)
        rec(3)
        if self.R:
            gp.gp_score_and_working_set(wl.q, wl.qstate, wl.slot_ids, wl.req_idx, self.cache,
                                        wl.block_tables, wl.context_lens, wl.positions,
                                        wl.rope_theta, wl.p, wl.sm_scale, self.C_max,
                                        a_short=self.a_s, a_long=self.a_l, ws_counts=self.wsc,
                                        n_cand=self.ncand, workspace=self.sws)
            rec(4)
            gp.gp_compact_or_grow(wl.req_idx, self.a_s, self.a_l, self.wsc, self.ncand, wl.tau,
                                  wl.k_loc, 0, self.cache, wl.block_tables, wl.n_pages,
                                  wl.context_lens, wl.refcount, wl.free_stack, wl.free_top,
                                  policies=self.policies, decision=self.dec,
                                  kept_idx=self.kept, workspace=self.cws)
        rec(5)

    # events of an overlapped step: main stream 0 start, 1 restored, 3 decoded, 8 compaction
    # moved (end); second stream 4 start, 5 summaries of the boundary requests, 6 scored,
    # 7 compress-or-grow planned
    NEV_OVERLAP = 9

    def step_overlap(self, ev=None):
        """GrowPage's overlap of the boundary pass with decoding. The main stream decodes every
        request from a copy of the block tables and lengths, with the summary update of the
        requests that are not at a boundary fused in and a grid that leaves compute units free;
        the second stream meanwhile updates the boundary requests' summaries, scores them and
        plans their compress-or-grow (decisions, pages, kept tokens: bookkeeping on the live
        tables only). The planned K/V movement runs on the main stream after the decode has read
        every page, with the whole GPU."""
        wl, gp, torch = self.wl, self.gp, self.torch
        main = torch.cuda.current_stream()
        sb = self.stream_b
        rec = (lambda k, st: ev[k] is not None and ev[k].record(st)) if ev is not None else (lambda k, st: None)
        rec(0, main)
        self.meta.copy_(self.meta0)
        rec(1, main)
        self.ev_a.record(main)
        gp.gp_paged_decode_attn_ex(wl.q, self.cache, self.bt_dec, self.ctx_dec, wl.max_context,
                                   wl.sm_scale, summaries=self.upd_main,
                                   max_workgroups=self.max_wg, out=self.out, lse=self.lse,
                                   workspace=self.dws)
        rec(3, main)
        with torch.cuda.stream(sb):
            sb.wait_event(self.ev_a)
            rec(4, sb)
            gp.gp_update_query_summaries(wl.q, self.slot_b, self.fresh0, wl.qstate, wl.beta_s,
                                         wl.beta_l)
            rec(5, sb)
            gp.gp_score_and_working_set(wl.q, wl.qstate, wl.slot_ids, wl.req_idx, self.cache,
                                        wl.block_tables, wl.context_lens, wl.positions,
                                        wl.rope_theta, wl.p, wl.sm_scale, self.C_max,
                                        a_short=self.a_s, a_long=self.a_l, ws_counts=self.wsc,
                                        n_cand=self.ncand, workspace=self.sws)
            rec(6, sb)
            self._compact(gp.growpage.PHASE_PLAN)
            rec(7, sb)
            self.ev_b.record(sb)
        main.wait_event(self.ev_b)
        self._compact(gp.growpage.PHASE_MOVE)
        rec(8, main)

    # events of a score-first step: main stream 0 start, 1 restored, 2 summaries of the boundary
    # requests, 3 scored, 4 decoded, 7 compaction moved (end); second stream 5 start, 6 planned
    NEV_SCORE_FIRST = 8

    def step_score_first(self, ev=None):
        """The boundary pass's latency-bound part first, alone, then decoding beside the rest.
        The main stream updates the boundary requests' summaries and scores them (their working
        sets: serial reductions that slow down several-fold beside a decode that keeps HBM's
        queues full), then decodes every request from a copy of the block tables and lengths with
        the other requests' summary update fused in; the second stream plans the compress-or-grow
        beside the decode (decisions, pages, kept tokens: bookkeeping on the live tables only);
        the planned K/V movement runs on the main stream after the decode."""
        wl, gp, torch = self.wl, self.gp, self.torch
        main = torch.cuda.current_stream()
        sb = self.stream_b
        rec = (lambda k, st: ev[k] is not None and ev[k].record(st)) if ev is not None else (lambda k, st: None)
        rec(0, main)
        self.meta.copy_(self.meta0)
        rec(1, main)
        gp.gp_update_query_summaries(wl.q, self.slot_b, self.fresh0, wl.qstate, wl.beta_s,
                                     wl.beta_l)
        rec(2, main)
        gp.gp_score_and_working_set(wl.q, wl.qstate, wl.slot_ids, wl.req_idx, self.cache,
                                    wl.block_tables, wl.context_lens, wl.positions,
                                    wl.rope_theta, wl.p, wl.sm_scale, self.C_max,
                                    a_short=self.a_s, a_long=self.a_l, ws_counts=self.wsc,
                                    n_cand=self.ncand, workspace=self.sws)
        rec(3, main)
        self.ev_a.record(main)
        gp.gp_paged_decode_attn_ex(wl.q, self.cache, self.bt_dec, self.ctx_dec, wl.max_context,
                                   wl.sm_scale, summaries=self.upd_main,
                                   max_workgroups=self.max_wg, out=self.out, lse=self.lse,
                                   workspace=self.dws)
        rec(4, main)
        with torch.cuda.stream(sb):
            sb.wait_event(self.ev_a)
            rec(5, sb)
            self._compact(gp.growpage.PHASE_PLAN)
            rec(6, sb)
            self.ev_b.record(sb)
        main.wait_event(self.ev_b)
        self._compact(gp.growpage.PHASE_MOVE)
        rec(7, main)

    def _compact(self, phases):
        wl, gp = self.wl, self.gp
        gp.gp_compact_or_grow(wl.req_idx, self.a_s, self.a_l, self.wsc, self.ncand, wl.tau,
                              wl.k_loc, 0, self.cache, wl.block_tables, wl.n_pages,
                              wl.context_lens, wl.refcount, wl.free_stack, wl.free_top,
                              policies=self.policies, decision=self.dec, kept_idx=self.kept,
                              workspace=self.cws, phases=phases)


def algorithmic_bytes(wl, path, np):
    """Bytes each row must move at least once (HBM), per step. decode_main is the decode call
    (all requests); summaries_main the summary updates fused into it (in the overlapped step, the
    requests that are not at a boundary)."""
    es = 4 if wl.dtype == "f32" else 2
    B, H_q, d, H_kv, b = wl.B, wl.H_q, wl.d, wl.H_kv, wl.page_size
    ctx = wl.context_lens.cpu().numpy().astype(np.int64)
    req = set(wl.req_idx.cpu().tolist()) if path.R else set()
    kv_r = np.zeros(B, dtype=np.int64)
    if wl.mixed:
        tags = wl.page_tag.cpu().numpy()
        bt = wl.block_tables.cpu().numpy()
        for r in range(B):
            n = int(ctx[r])
            t = tags[bt[r, np.arange(n) // b]]
            kv_r[r] = (int((t == 2).sum()) * H_kv * d * 2 * 2             # bf16 K + V
                       + int((t == 1).sum()) * H_kv * (d * 2 + 2 * 4)     # fp8 K + V codes + 2 scales
                       + int((t == 3).sum()) * H_kv * (d + 2 * 2))        # INT4 K + V codes + 2 scales
    else:
        kv_r[:] = ctx * H_kv * d * es * 2
    pages_r = np.array([math.ceil(c / b) for c in ctx], dtype=np.int64)
    per_req = kv_r + 2 * H_q * d * es + H_q * 4 + pages_r * 4 + 4
    summ_r = H_q * d * (es + 4 * 4) + 5   # q_pre read, both fp32 summaries read and written
    n_summ = B - len(req) if path.overlap else B   # the decode call's fused updates
    out = dict(decode=int(per_req.sum()), decode_kv=int(kv_r.sum()),
               decode_main=int(per_req.sum()), decode_main_kv=int(kv_r.sum()),
               summaries=B * summ_r, summaries_main=n_summ * summ_r, score=0, compact=0)
    for r in req:
        c = max(0, (math.ceil(int(ctx[r]) / b) - 1) * b)
        out["score"] += c * H_kv * d * es + 4 * H_kv * c * 4
    return out


def moved_bytes(wl, path, ctx_before, np):
    """K/V bytes read and written by the last step's compaction (tokens that shifted)."""
    if not path.R:
        return 0
    es = 4 if wl.dtype == "f32" else 2
    kept = path.kept.cpu().numpy()
    dec = path.dec.cpu().numpy()
    nc = path.ncand.cpu().numpy()
    ctx_after = wl.context_lens.cpu().numpy()
    req = wl.req_idx.cpu().tolist()
    tot = 0
    for i, r in enumerate(req):
        if dec[i] not in (0, 2) or ctx_after[r] == ctx_before[r]:
            continue
        for h in range(wl.H_kv):
            row = kept[i, h, :nc[i]]
            same = np.nonzero(row != np.arange(len(row)))[0]
            first = int(same[0]) if len(same) else int(ctx_after[r])
            tot += (int(ctx_after[r]) - first) * wl.d * es * 2 * 2   # K and V, read + write
    return tot


def int4_leg(wl, gp, torch, np, steps):
    """Decode of the same batch with every used page demoted to INT4 (one quantiser call over
    all of them, timed once), on a mixed cache sharing the bf16 pools. Returns a dict with the
    decode time per launch and its algorithmic bytes: codes d/2 bytes per K and per V row plus
    two half scales per token and KV head."""
    dev = wl.k_pool.device
    P, H, b, d = wl.k_pool.shape
    tiny = torch.zeros(64, dtype=torch.uint8, device=dev)  # fp8 pools: no page carries that tag
    cache = gp.KVCache(wl.k_pool, wl.v_pool, b, k8=tiny, v8=tiny, k_scale=tiny.view(torch.float32),
                       v_scale=tiny.view(torch.float32),
                       page_tag=torch.full((P,), 2, dtype=torch.uint8, device=dev),
                       k4=torch.empty((P, H, b, d // 2), dtype=torch.uint8, device=dev),
                       v4=torch.empty((P, H, b // 4, d, 2), dtype=torch.uint8, device=dev),
                       k4_scale=torch.empty((P, H, b), dtype=torch.float16, device=dev),
                       v4_scale=torch.empty((P, H, b), dtype=torch.float16, device=dev))
    bt = wl.block_tables.cpu().numpy()
    used = torch.as_tensor(np.unique(bt[bt >= 0]), dtype=torch.int32, device=dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    gp.gp_quantize_pages_int4(cache, used)
    e[1].record()
    need = gp.gp_paged_decode_attn_workspace_size(wl.B, wl.H_q, H, d, b, wl.max_context)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty_like(wl.q)
    lse = torch.empty((wl.B, wl.H_q), dtype=torch.float32, device=dev)

    def run():
        gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens, wl.max_context,
                                wl.sm_scale, out=out, lse=lse, workspace=ws)

    def timed():
        for _ in range(3):
            run()
        e[2].record()
        for _ in range(steps):
            run()
        e[3].record()
        torch.cuda.synchronize()
        return e[2].elapsed_time(e[3]) / steps
    # every page the tables reach is INT4 and the cache says so: the bf16 / fp8 pass, which would
    # find no page, is not launched (gp_kv_cache.tags_present); the same call with the tags
    # undeclared runs both passes
    cache.tags_present = (gp.growpage.TAG_INT4,)
    ms = timed()
    cache.tags_present = ()
    ms_both = timed()
    ctx = wl.context_lens.cpu().numpy().astype(np.int64)
    pages = np.array([math.ceil(c / b) for c in ctx], dtype=np.int64)
    kv = int(ctx.sum()) * H * (d + 2 * 2)
    total = kv + int((2 * wl.H_q * d * 2 + wl.H_q * 4 + pages * 4 + 4).sum())
    return dict(pages=int(used.numel()), quantize_ms=round(e[0].elapsed_time(e[1]), 4),
                decode_ms=round(ms, 4), tags_declared=True, decode_ms_tags_undeclared=round(ms_both, 4),
                bytes_per_launch=total,
                achieved_gbps=round(total / (ms * 1e-3) / 1e9, 1),
                frac=round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4))


BOUNDARY_CASES = (("long_reasoning_d128", 16), ("long_reasoning_d64", 16), ("long_reasoning_d128", 256),
                  ("long_reasoning_d64", 256), ("prefix_shared", 16), ("tiny", 16),
                  ("mixed_precision", 16))
MIXED_BOUNDARY = ("mixed-precision pages, 40/30/30 fp8/bf16/INT4 with none released (B=128, ctx "
                  "U[8192,24576], Hq=32, Hkv=8, d=128, b=16), 16 seeded requests forced to compress")
MIXED_NAMES = ("k8", "v8", "k_scale", "v_scale", "k4", "v4", "k4_scale", "v4_scale")


def boundary_leg(name, b, gp, torch, np, reps, make_workload):
    """Boundary-pass latency per request (score + working set, then compress-or-grow with every
    boundary request forced to compress, so each one moves its tokens) on workload `name` with
    `b`-token pages. The integer page state and the boundary requests' K/V pages are restored
    before every repetition, outside the timed region; the median of `reps` after 3 warmups, with
    two events around the whole pass (the score / compress-or-grow split comes from a second
    series with a marker between the two calls). Also the same pass for the first boundary request
    alone (R = 1). Each call passes the
    candidate bound of its own requests (C_max from their lengths, which the caller knows), as the
    step does. Bytes per request: keys of C read, both score planes written and read back, and the
    K/V of the tokens that shift, read and written."""
    dev = "cuda:0"
    wl = make_workload(name, "full", device=dev, page_size=b)
    if wl.mixed:
        # the mixed-precision batch with its pages re-tagged fp8 / bf16 / INT4 (a request
        # holding a released page is not compacted) and 16 seeded requests, forced to compress
        from workloads.configs import attach_mixed_pools
        rng = np.random.Generator(np.random.PCG64(2024))
        tags = rng.choice([1, 2, 3], size=wl.num_pages, p=[0.4, 0.3, 0.3]).astype(np.uint8)
        attach_mixed_pools(wl, tags, seed=5)
        wl.req_idx = torch.as_tensor(np.sort(rng.choice(wl.B, size=16, replace=False)),
                                     dtype=torch.int32, device=dev)
    if name == "prefix_shared":
        # the prefix-shared batch's 8 requests that its own policy compresses (the other 8 grow)
        keep = [k for k, pol in enumerate(wl.req_policy) if pol == 1]
        wl.req_idx = wl.req_idx[keep].contiguous()
        wl.req_policy = [wl.req_policy[k] for k in keep]
    path = Path(wl, gp, torch)
    path.build_state()
    es = 4 if wl.dtype == "f32" else 2
    names = ("block_tables", "n_pages", "context_lens", "refcount", "free_stack", "free_top")
    ints = {n: getattr(wl, n).clone() for n in names}
    req_all = wl.req_idx.clone()
    bt = wl.block_tables.cpu().numpy()
    pages = np.unique(bt[req_all.cpu().numpy()][bt[req_all.cpu().numpy()] >= 0])
    pidx = torch.as_tensor(pages, dtype=torch.long, device=dev)
    pools = ("k_pool", "v_pool") + (MIXED_NAMES if wl.mixed else ())
    saved = {n: getattr(wl, n).index_select(0, pidx) for n in pools}
    tag0 = wl.page_tag.clone() if wl.mixed else None
    out = {}

    def restore():
        for n in names:
            getattr(wl, n).copy_(ints[n])
        for n in pools:
            getattr(wl, n).index_copy_(0, pidx, saved[n])
        if tag0 is not None:
            wl.page_tag.copy_(tag0)

    ctx_h = ints["context_lens"].cpu().tolist()
    for label, req in (("all", req_all), ("one", req_all[:1].clone())):
        R = req.numel()
        pol = torch.full((R,), 1, dtype=torch.int32, device=dev)   # forced compress
        # the candidate bound of this call, from the lengths the caller knows (as in the step)
        cm = max(max(0, (math.ceil(ctx_h[r] / b) - 1) * b) for r in req.cpu().tolist())
        C = max(16, -(-cm // 16) * 16)
        a_s = torch.empty((R, wl.H_kv, C), dtype=torch.float32, device=dev)
        a_l = torch.empty_like(a_s)
        kept_t = torch.empty((R, wl.H_kv, C), dtype=torch.int32, device=dev)

        def score():
            gp.gp_score_and_working_set(wl.q, wl.qstate, wl.slot_ids, req, path.cache,
                                        wl.block_tables, wl.context_lens, wl.positions,
                                        wl.rope_theta, wl.p, wl.sm_scale, C,
                                        a_short=a_s, a_long=a_l,
                                        ws_counts=path.wsc[:R], n_cand=path.ncand[:R],
                                        workspace=path.sws)

        def compact():
            gp.gp_compact_or_grow(req, a_s, a_l, path.wsc[:R], path.ncand[:R],
                                  wl.tau, wl.k_loc, 0, path.cache, wl.block_tables, wl.n_pages,
                                  wl.context_lens, wl.refcount, wl.free_stack, wl.free_top,
                                  policies=pol, decision=path.dec[:R], kept_idx=kept_t,
                                  workspace=path.cws)

        def timed(run_score, run_compact, split):
            # split: a marker between the two calls gives the score / compress-or-grow split,
            # at the cost of the marker's own gap; the whole pass is timed without it
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            t_s, t_c = [], []
            for it in range(reps + 3):
                restore()
                ev[0].record()
                run_score()
                if split:
                    ev[1].record()
                run_compact()
                ev[2].record()
                torch.cuda.synchronize()
                if it >= 3:
                    if split:
                        t_s.append(ev[0].elapsed_time(ev[1]))
                        t_c.append(ev[1].elapsed_time(ev[2]))
                    else:
                        t_s.append(ev[0].elapsed_time(ev[2]))
            return float(np.median(t_s)), float(np.median(t_c)) if t_c else 0.0

        ms_s, ms_c = timed(score, compact, True)
        ms_pass, _ = timed(score, compact, False)
        dec = path.dec[:R].cpu().numpy()
        nc = path.ncand[:R].cpu().numpy().astype(np.int64)
        kept = kept_t.cpu().numpy()
        ctx0 = ints["context_lens"].cpu().numpy()
        ctx1 = wl.context_lens.cpu().numpy()
        moved = 0
        # bytes of one token row of K or V by page tag (mixed pages: codes plus row scale)
        row_bytes = {1: wl.d + 4, 2: wl.d * 2, 3: wl.d // 2 + 2}
        bt0 = ints["block_tables"].cpu().numpy()
        bt1 = wl.block_tables.cpu().numpy()
        t0 = tag0.cpu().numpy() if tag0 is not None else None
        t1 = wl.page_tag.cpu().numpy() if tag0 is not None else None
        for i, r in enumerate(req.cpu().tolist()):
            if dec[i] not in (0, 2, 4) or ctx1[r] == ctx0[r]:
                continue
            firsts = []
            for h in range(wl.H_kv):
                row = kept[i, h, :nc[i]]
                diff = np.nonzero(row != np.arange(len(row)))[0]
                firsts.append(int(diff[0]) if len(diff) else int(ctx1[r]))
            if t0 is None:
                moved += sum(int(ctx1[r]) - f for f in firsts) * wl.d * es * 2 * 2
                continue
            # mixed pages: every head rewrites from the first changed page (read in the
            # source page's format, written in the destination page's)
            j0 = min(firsts) // b * b
            for j in range(j0, int(ctx1[r])):
                rd = row_bytes[int(t0[bt0[r, j // b]])]
                wr = row_bytes[int(t1[bt1[r, j // b]])]
                moved += (rd + wr) * 2 * wl.H_kv
        score_bytes = 0
        for i, r in enumerate(req.cpu().tolist()):
            c = int(nc[i])
            if t0 is None:
                score_bytes += c * wl.H_kv * wl.d * es
            else:   # keys of C in their pages' formats (released pages are not read)
                tg = t0[bt0[r, np.arange(c) // b]] if c else np.zeros(0, np.uint8)
                score_bytes += int(sum(row_bytes.get(int(t), 0) for t in tg)) * wl.H_kv
            score_bytes += 4 * wl.H_kv * c * 4          # both score planes written and read
        byts = score_bytes + moved
        ms = ms_pass
        out[label] = dict(requests=int(R), us_per_request=round(ms * 1e3 / R, 1),
                          score_us=round(ms_s * 1e3, 1), compact_us=round(ms_c * 1e3, 1),
                          bytes=byts, gbps=round(byts / (ms * 1e-3) / 1e9, 1),
                          mean_candidates=round(float(nc.mean()), 1), c_max=C,
                          decisions=sorted(set(int(x) for x in dec)))
    res = dict(workload=MIXED_BOUNDARY if wl.mixed else WORKLOAD_NAMES[name], page_size=b,
               k_loc=int(wl.k_loc), **out["all"], single_request=out["one"])
    del wl, path, saved
    torch.cuda.empty_cache()
    return res


DECODE_CASES = ("tiny", "long_reasoning_d64", "long_reasoning_d128", "prefix_shared", "mixed_precision")


def decode_leg(name, gp, torch, np, reps, make_workload):
    """One decode call over the whole batch of workload `name` (16-token pages, no grid cap, no
    fused update), the median of `reps` after 3 warmups with HIP events on the launching stream.
    Bytes on the decode's byte model: K/V of every visible token in its page's format (released
    pages none), Q, O, lse, block-table entries, lengths. The prefix-shared batch also reports
    its unique bytes: each shared token once, as HBM must supply it."""
    dev = "cuda:0"
    wl = make_workload(name, "full", device=dev)
    cache = gp.KVCache.from_workload(wl)
    if wl.mixed:
        # the tags the batch's pages carry, as a caller that manages its tiers knows them: a
        # decode pass with none of its tags is not launched (gp_kv_cache.tags_present)
        bt = wl.block_tables.cpu().numpy()
        cache.tags_present = tuple(int(t) for t in np.unique(wl.page_tag.cpu().numpy()[np.unique(bt[bt >= 0])]))
    B, H_q, d = wl.q.shape
    out = torch.empty_like(wl.q)
    lse = torch.empty((B, H_q), dtype=torch.float32, device=dev)
    n = gp.gp_paged_decode_attn_workspace_size(B, H_q, wl.H_kv, d, wl.page_size, wl.max_context)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    times = []
    for it in range(reps + 3):
        ev[0].record()
        gp.gp_paged_decode_attn(wl.q, cache, wl.block_tables, wl.context_lens, wl.max_context,
                                wl.sm_scale, out=out, lse=lse, workspace=ws)
        ev[1].record()
        torch.cuda.synchronize()
        if it >= 3:
            times.append(ev[0].elapsed_time(ev[1]))
    ms = float(np.median(times))

    class _NoBoundary:
        R = 0
        overlap = False
    by = algorithmic_bytes(wl, _NoBoundary, np)
    res = dict(workload=WORKLOAD_NAMES[name], batch=int(B),
               mean_context=round(float(wl.context_lens.float().mean()), 1),
               decode_ms=round(ms, 4), bytes=by["decode"], kv_bytes=by["decode_kv"],
               gbps=round(by["decode"] / (ms * 1e-3) / 1e9, 1),
               frac=round(by["decode"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4))
    if name == "prefix_shared":
        # shared prefix pages are read by every request; count each (page, slot) token once
        es = 2
        ctx = wl.context_lens.cpu().numpy().astype(np.int64)
        bt = wl.block_tables.cpu().numpy().astype(np.int64)
        b = wl.page_size
        toks = np.concatenate([bt[r, np.arange(c) // b] * b + np.arange(c) % b
                               for r, c in enumerate(ctx) if c > 0])
        uniq_kv = int(np.unique(toks).size) * wl.H_kv * d * es * 2
        uniq = by["decode"] - by["decode_kv"] + uniq_kv
        res.update(unique_bytes=uniq, unique_gbps=round(uniq / (ms * 1e-3) / 1e9, 1),
                   unique_frac=round(uniq / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4))
    del wl, cache, out, lse, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, path, budget_s, np):
    """The float64 oracle on a bounded sample: decode of whole requests, then the boundary pass
    of boundary requests, until the time budget is used. Returns GB/s on the same byte model."""
    import torch
    from oracle import attention as oatt
    from oracle import boundary as ob
    from oracle import summaries as osum
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    b = wl.page_size
    es = 4 if wl.dtype == "f32" else 2
    ctx = wl.context_lens.cpu().numpy().astype(np.int64)
    bt_all = wl.block_tables.cpu().numpy().astype(np.int64)

    def host_pages(reqs):
        rows = bt_all[reqs]
        pages = np.unique(rows[rows >= 0])
        idx = torch.as_tensor(pages, device=wl.k_pool.device, dtype=torch.long)
        remap = np.full(wl.num_pages, -1, dtype=np.int64)
        remap[pages] = np.arange(len(pages))
        sub = {"k": wl.k_pool.index_select(0, idx).cpu().double().numpy(),
               "v": wl.v_pool.index_select(0, idx).cpu().double().numpy()}
        if wl.mixed:
            for nm in MIXED_POOLS:
                sub[nm] = getattr(wl, nm).index_select(0, idx).cpu().numpy()
        bt = np.where(rows >= 0, remap[np.maximum(rows, 0)], -1)
        return sub, bt

    t_used, bytes_done = 0.0, 0
    qst0 = wl.qstate.cpu().double().numpy()
    q64 = wl.q.cpu().double().numpy()

    def one_pass(budget_left):
        """Summary update, decode request by request, then the boundary pass; returns the time,
        the bytes and what the pass covered."""
        t, nbytes, what = 0.0, 0, []
        qst = qst0.copy()
        t0 = time.perf_counter()
        osum.update_query_summaries(q64, wl.slot_ids.cpu().numpy(), [False] * wl.B, qst,
                                    wl.beta_s, wl.beta_l)
        t += time.perf_counter() - t0
        nbytes += wl.B * wl.H_q * wl.d * (es + 16)
        what.append(f"summary update of all {wl.B} requests")
        n_dec = 0
        for r in range(wl.B):
            if t > 0.6 * budget_left:
                break
            sub, bt = host_pages([r])
            extra = {}
            if wl.mixed:
                extra = {nm: sub[nm] for nm in MIXED_POOLS}
            t0 = time.perf_counter()
            oatt.paged_decode_attn(q64[r:r + 1], sub["k"], sub["v"], bt, ctx[r:r + 1], b,
                                   wl.sm_scale, **extra)
            t += time.perf_counter() - t0
            nbytes += int(ctx[r]) * wl.H_kv * wl.d * es * 2
            n_dec += 1
        what.append(f"decode of {n_dec} of {wl.B} requests")
        n_bnd = 0
        if path.R and not wl.mixed:
            req = wl.req_idx.cpu().tolist()
            for i, r in enumerate(req):
                if t > budget_left:
                    break
                sub, bt = host_pages([r])
                t0 = time.perf_counter()
                a_s, a_l, ws, nc = ob.score_and_working_set(
                    q64[r:r + 1], qst, wl.slot_ids[r:r + 1].cpu().numpy(), [0], sub["k"], bt,
                    ctx[r:r + 1], wl.positions[r:r + 1].cpu().numpy(), b, wl.rope_theta, wl.p,
                    wl.sm_scale)
                st = dict(bt=bt.copy(), n_pages=wl.n_pages[r:r + 1].cpu().numpy().astype(np.int64),
                          ctx=ctx[r:r + 1].copy(), rc=np.ones(sub["k"].shape[0], dtype=np.int64),
                          fs=np.full(sub["k"].shape[0] + 1, -1, dtype=np.int64),
                          top=np.zeros(1, dtype=np.int64))
                ob.compact_or_grow([0], a_s, a_l, ws, nc, wl.tau, wl.k_loc, ob.POLICY_FORCE_COMPRESS,
                                   sub["k"], sub["v"], st["bt"], st["n_pages"], st["ctx"], st["rc"],
                                   st["fs"], st["top"], b, policies=[ob.POLICY_FORCE_COMPRESS])
                t += time.perf_counter() - t0
                c = int(nc[0])
                nbytes += c * wl.H_kv * wl.d * es + 4 * wl.H_kv * c * 4
                n_bnd += 1
            what.append(f"boundary pass (score, working set, forced compress) of {n_bnd} of "
                        f"{len(req)} boundary requests")
        return t, nbytes, what

    # whole passes over the step while another one fits the budget (a pass that the budget cuts
    # short covers part of the step and is the only one)
    passes, what = 0, []
    while True:
        t, nbytes, w = one_pass(budget_s - t_used)
        t_used += t
        bytes_done += nbytes
        passes += 1
        what = w
        if t_used + t > budget_s:
            break
    what = what + [f"{passes} pass{'es' if passes > 1 else ''}"]
    gbps = bytes_done / t_used / 1e9 if t_used > 0 else None
    return dict(value=gbps, unit="GB/s", cores=int(blas), kind="oracle",
                sample="; ".join(what) + f"; {t_used:.1f} s of oracle time, bytes on the "
                       "same algorithmic model as value (numpy float64; BLAS threads = cores, "
                       "elementwise numpy single-threaded)",
                seconds=round(t_used, 2))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import paged_kv_cache_472_amd as gp
    from workloads import make_workload

    gp.lib()  # raises if the HIP library is missing: there is no other path
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    print(f"[bench] building workload {args.workload} on {dev}", file=sys.stderr, flush=True)
    wl = make_workload(args.workload, "full", device=dev)
    path = Path(wl, gp, torch, overlap=args.overlap, reserve_cus=args.reserve_cus)
    path.build_state()
    torch.cuda.synchronize()
    ctx_before = wl.context_lens.cpu().numpy().copy()

    step = {0: path.step, 1: path.step_overlap, 2: path.step_score_first}[path.mode]
    nev = {0: 6, 1: Path.NEV_OVERLAP, 2: Path.NEV_SCORE_FIRST}[path.mode]
    print(f"[bench] warmup {args.warmup} (overlap {int(path.overlap)})", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed steps record only the two events around the main decode call (the roofline's):
    # every other event adds a marker between the step's launches (about 11 us per step in all).
    # The per-row breakdown comes from a second run of the same steps with every event.
    dec_a, dec_z = {0: (2, 3), 1: (1, 3), 2: (3, 4)}[path.mode]
    timed = [[torch.cuda.Event(enable_timing=True) if j in (dec_a, dec_z) else None
              for j in range(nev)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(timed[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    dec_ms = sum(timed[k][dec_a].elapsed_time(timed[k][dec_z]) for k in range(args.steps)) / args.steps
    # K/V the last timed step's compaction moved (pages keep what earlier steps wrote, so the
    # amount drifts a little from step to step)
    moved = moved_bytes(wl, path, ctx_before, np)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    print(f"[bench] per-row breakdown, {args.steps} instrumented steps", file=sys.stderr, flush=True)
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()

    def avg_ms(a, z):
        return sum(events[k][a].elapsed_time(events[k][z]) for k in range(args.steps)) / args.steps

    # the summary update runs inside the decode call (events 1 and 2 are adjacent)
    if path.mode == 2:
        rows_ms = dict(restore=avg_ms(0, 1), boundary_summaries=avg_ms(1, 2),
                       score_and_working_set=avg_ms(2, 3), paged_decode_attn_with_summaries=avg_ms(3, 4),
                       compact_or_grow_plan=avg_ms(5, 6), compact_or_grow_move_incl_wait=avg_ms(4, 7))
        event_step_ms = avg_ms(0, 7)
    elif path.overlap:
        rows_ms = dict(restore=avg_ms(0, 1), paged_decode_attn_with_summaries=avg_ms(1, 3),
                       boundary_summaries=avg_ms(4, 5), score_and_working_set=avg_ms(5, 6),
                       compact_or_grow_plan=avg_ms(6, 7), compact_or_grow_move_incl_wait=avg_ms(3, 8))
        event_step_ms = avg_ms(0, 8)
    else:
        rows_ms = dict(restore=avg_ms(0, 1), paged_decode_attn_with_summaries=avg_ms(2, 3))
        if path.R:
            rows_ms["score_and_working_set"] = avg_ms(3, 4)
            rows_ms["compact_or_grow"] = avg_ms(4, 5)
        event_step_ms = avg_ms(0, 5)

    single = None
    if path.overlap:
        # the same rows one after another on one stream, for reference
        print(f"[bench] single-stream reference, {args.steps} steps", file=sys.stderr, flush=True)
        # (timed with the decode bracket only, like the main steps; rows from a second run)
        tm1 = [[torch.cuda.Event(enable_timing=True) if j in (2, 3) else None for j in range(6)]
               for _ in range(args.steps)]
        for _ in range(2):
            path.step()
        torch.cuda.synchronize()
        s0 = time.perf_counter()
        for k in range(args.steps):
            path.step(tm1[k])
        torch.cuda.synchronize()
        ms1 = (time.perf_counter() - s0) * 1e3 / args.steps
        dec1 = sum(tm1[k][2].elapsed_time(tm1[k][3]) for k in range(args.steps)) / args.steps
        ev1 = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
        for k in range(args.steps):
            path.step(ev1[k])
        torch.cuda.synchronize()
        a1 = lambda i, j: sum(ev1[k][i].elapsed_time(ev1[k][j]) for k in range(args.steps)) / args.steps  # noqa: E731
        single = dict(ms_per_step=round(ms1, 4), decode_ms=round(dec1, 4),
                      score_us=round(a1(3, 4) * 1e3, 1), compact_us=round(a1(4, 5) * 1e3, 1),
                      boundary_us_per_request=round((a1(3, 5)) * 1e3 / path.R, 1))

    by = algorithmic_bytes(wl, path, np)
    by["compact"] = moved
    step_bytes = by["decode"] + by["summaries"] + by["score"] + by["compact"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    if single is not None:
        single["value"] = round(step_bytes / (single["ms_per_step"] * 1e-3) / 1e9, 2)
        # the same decode call with the GPU to itself (no grid cap, two tiles in flight per wave)
        dec_gbps = (by["decode_main"] + by["summaries"]) / (single["decode_ms"] * 1e-3) / 1e9
        single["decode_gbps"] = round(dec_gbps, 1)
        single["decode_frac"] = round(dec_gbps / HBM_PEAK_GBPS, 4)

    achieved = (by["decode_main"] + by["summaries_main"]) / (dec_ms * 1e-3) / 1e9

    # plain device copy of known size: the practical HBM ceiling on this machine
    nbytes = int(args.copy_probe_gib * (1 << 30))
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    traffic = None
    if os.path.exists(PMC_FILE):
        with open(PMC_FILE) as fh:
            pmc = json.load(fh)
        if (pmc.get("decode_src_sha") == file_sha(DECODE_SRC) and pmc.get("workload") == args.workload
                and pmc.get("overlap", 0) == int(path.overlap)
                and pmc.get("reserve_cus", 0) == (args.reserve_cus if path.overlap else 0)
                and pmc.get("decode_call") == "every request, fused summary update"):
            traffic = pmc.get("bytes_per_launch")

    int4 = None
    if args.int4 and not wl.mixed and wl.dtype == "bf16":
        print("[bench] INT4 leg: demote every used page, time decode", file=sys.stderr, flush=True)
        int4 = int4_leg(wl, gp, torch, np, args.steps)
        # against the same batch in bf16 decoded with the full grid
        ref_ms = single["decode_ms"] if single is not None else dec_ms
        int4["speedup_vs_bf16_decode"] = round(ref_ms / int4["decode_ms"], 3)

    boundary = None
    if path.R:
        cmp_ms = rows_ms.get("compact_or_grow")
        if cmp_ms is None:
            cmp_ms = rows_ms["compact_or_grow_plan"] + rows_ms["compact_or_grow_move_incl_wait"]
        bnd_ms = rows_ms["score_and_working_set"] + cmp_ms
        boundary = dict(requests=path.R, us_per_request=bnd_ms * 1e3 / path.R,
                        score_us=rows_ms["score_and_working_set"] * 1e3,
                        compact_us=cmp_ms * 1e3, decisions=path.dec.cpu().tolist())

    bpass = None
    if args.boundary_pass:
        bpass = []
        for name, b in BOUNDARY_CASES:
            print(f"[bench] boundary pass on workload {name}, {b}-token pages", file=sys.stderr,
                  flush=True)
            bpass.append(boundary_leg(name, b, gp, torch, np, 20, make_workload))

    dconf = None
    if args.decode_configs:
        dconf = []
        for name in DECODE_CASES:
            print(f"[bench] decode of workload {name}", file=sys.stderr, flush=True)
            dconf.append(decode_leg(name, gp, torch, np, 20, make_workload))

    cpu = None
    if args.cpu_seconds > 0:
        print(f"[bench] cpu_baseline (oracle, ~{args.cpu_seconds:.0f} s)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(wl, path, args.cpu_seconds, np)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if wl.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[args.workload], "batch": wl.B,
                   "mean_context": round(float(wl.context_lens.float().mean()), 1),
                   "boundary_requests": path.R, "page_size": wl.page_size},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "paged_decode_attn_ex (stream-K decode of every request with the "
                               "fused summary update + merge launches)" + (
                         ", grid capped, beside the boundary pass on a second stream"
                         if path.overlap else ""),
                     "bytes_per_launch": by["decode_main"] + by["summaries_main"],
                     "avg_launch_ms": round(dec_ms, 4)},
        "cpu_baseline": cpu,
        "value_is": "whole-step throughput: algorithmic bytes of every row of the step (decode "
                    "K/V, Q/O, tables and lse, summaries, score keys and planes, compaction "
                    "moves) / step time; the decode alone is decode_kv_gbps",
        "decode_kv_gbps": round(by["decode_main_kv"] / (dec_ms * 1e-3) / 1e9, 1),
        "decode_kv_frac": round(by["decode_main_kv"] / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "overlap": int(path.overlap),
        "decode_frac_of_copy": round(achieved / copy_gbps, 4),
        "copy_gbps": round(copy_gbps, 1),
        "boundary": boundary,
        "boundary_pass": bpass,
        "int4_decode": int4,
        "decode_configs": dconf,
        "single_stream": single,
        "rows_ms": {k: round(v, 4) for k, v in rows_ms.items()},
        "event_ms_per_step": round(event_step_ms, 4),
        "bytes_per_step": by,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
