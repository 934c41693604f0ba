"""Helpers for the GPU parity tests (HIP library through the C ABI vs the CPU oracle)."""
import sys

import numpy as np
import torch

from workloads import make_workload

TOL = {"f32": 2e-4}
DEV = "cuda:0"

# fp32 outputs (lse, scores, summaries) are checked at the fp32 bound whatever the cache dtype.
# lse: the logits of bf16 / fp8 / INT4 keys against bf16 (or exactly half-rounded) queries are
# exact products summed in fp32; the running sum of exponentials adds at most one fp32 rounding
# per 16-token tile, so its relative error stays below 2048 * 2^-24 = 1.2e-4 even for 32K tokens,
# and lse inherits it as an absolute error.
LSE_TOL = 2e-4
# bf16 outputs: the probabilities are rounded to bf16 (fp8 pages: times the row scale; INT4
# pages: to half, toward zero) before the value product, and the output once more at the end.
# bf16 keeps 8 significant bits, so each rounding is a relative error of at most 2^-8:
# |out - ref| <= 2^-8 |ref| + 2^-8 sum_j w_j |v_j| (+ fp32 accumulation). The bound below doubles
# both terms; A = sum_j w_j |v_j| is the oracle's attention over |V|.
OUT_REL_BF16 = 2.0 ** -7
OUT_ABS_BF16 = 1e-5
# scores: the summaries meet bf16 keys as a hi + lo bf16 pair (16 significant bits), so a logit
# is off by at most about 2^-16 sum_i |q_i k_i| / sqrt(d) (~1e-4 for RMS-1 queries and N(0,1)
# keys); that moves every weight by the same relative amount. Bound: 1e-3 relative, plus a
# floor of 1e-6 of the row's largest weight for weights the GPU flushes to zero.
SCORE_REL = 1e-3
SCORE_FLOOR = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# largest observed errors of the session, printed by the terminal summary (tests/conftest.py)
WORST = {}


def note_worst(name, value, bound, where):
    if name not in WORST or value > WORST[name][0]:
        WORST[name] = (value, bound, where)


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


def decode_reference(q, k_pool, v_pool, block_tables, context_lens, page_size, sm_scale,
                     mixed=None):
    """The oracle's decode (out, lse) of every request, plus its attention over |V| (the
    probability-weighted mean of |v| that scales the bf16 rounding bound)."""
    from oracle import attention as oatt
    q = np.asarray(q, dtype=np.float64)
    B, H_q, d = q.shape
    H_kv = np.asarray(k_pool).shape[1]
    G = H_q // H_kv
    out = np.zeros((B, H_q, d))
    lse = np.zeros((B, H_q))
    wabs = np.zeros((B, H_q, d))
    mx = mixed or {}
    for r in range(B):
        k, v, _ = oatt.gather_request_kv(r, k_pool, v_pool, block_tables, context_lens,
                                         page_size, **mx)
        for h in range(H_kv):
            rows = slice(h * G, (h + 1) * G)
            out[r, rows], lse[r, rows] = oatt.attend(q[r, rows], k[h], v[h], sm_scale)
            wabs[r, rows], _ = oatt.attend(q[r, rows], k[h], np.abs(v[h]), sm_scale)
    return out, lse, wabs


def check_decode(out, lse, ref, dtype, label):
    """Element-wise check of a decode against decode_reference(): lse at the fp32 bound, out at
    2e-4 (fp32) or the bf16 rounding bound; prints the observed errors."""
    ref_o, ref_l, ref_a = ref
    o = out.detach().to("cpu", torch.float64).numpy() if isinstance(out, torch.Tensor) else out
    l_ = lse.detach().cpu().numpy() if isinstance(lse, torch.Tensor) else lse
    eo, nan_o = maxabs(o, ref_o)
    el, nan_l = maxabs(l_, ref_l)
    if dtype == "f32":
        bound = np.full(ref_o.shape, TOL["f32"])
    else:
        bound = OUT_REL_BF16 * (np.abs(ref_o) + ref_a) + OUT_ABS_BF16
    ratio = float(np.max(np.abs(o - ref_o) / bound)) if ref_o.size else 0.0
    say(f"[{label}] max|out-ref|={eo:.3e} (max error / bound {ratio:.3f}) "
        f"max|lse-ref|={el:.3e} (bound {LSE_TOL:.0e})")
    note_worst(f"decode lse ({dtype} cache)", el, LSE_TOL, label)
    note_worst(f"decode out, error / bound ({dtype} cache)", ratio, 1.0, label)
    assert not nan_o and not nan_l, "NaN in output or lse"
    assert el <= LSE_TOL, f"lse error {el:.3e}"
    assert ratio <= 1.0, f"out error {eo:.3e}, {ratio:.3f} of the bound"
    return eo, el


def check_scores(a, ref, n, label=""):
    """Scores of one request (rows [H_kv, >= n]) against the oracle's: relative bound plus a
    floor of the row maximum; returns the largest relative error."""
    a = np.asarray(a, dtype=np.float64)[:, :n]
    ref = np.asarray(ref, dtype=np.float64)[:, :n]
    assert not np.isnan(a).any(), f"NaN in scores {label}"
    if n == 0:
        return 0.0
    floor = SCORE_FLOOR * ref.max(axis=1, keepdims=True)
    err = np.abs(a - ref)
    assert (err <= SCORE_REL * np.abs(ref) + floor).all(), \
        f"scores {label}: max|a-ref| {err.max():.3e}, max rel {np.max(err / np.maximum(ref, 1e-300)):.3e}"
    big = ref > floor
    rel = float(np.max(err[big] / ref[big])) if big.any() else 0.0
    note_worst("score relative error", rel, SCORE_REL, label)
    return rel
