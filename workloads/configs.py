"""Seeded synthetic decode / page-boundary workloads.

Storage layout produced here (the layout the library consumes):

* ``k_pool``  ``[num_pages, H_kv, b, d]``   one page of one KV head is ``b`` key rows of ``d``.
* ``v_pool``  ``[num_pages, H_kv, d, b]``   values are stored transposed inside a page
  (``d`` rows of ``b`` tokens), so that the token index is the contiguous axis.
* mixed-precision pages (GrowPage's companion page on packed KV, PASK B.5, and the fp8 tag of
  the mixed-precision workload): ``k8 [num_pages, H_kv, b, d]`` and ``v8 [num_pages, H_kv, d, b]`` hold
  OCP E4M3FN codes, ``k_scale / v_scale [num_pages, H_kv, b]`` one fp32 scale per token row
  and KV head, and ``page_tag [num_pages]`` (0 released, 1 fp8, 2 bf16, 3 int4).
* INT4 pages (PASK B.5, present in every mixed workload): ``k4 [num_pages, H_kv, b, d/2]``
  (two signed nibbles per byte along d, even index low), ``v4 [num_pages, H_kv, b/4, d, 2]``
  (four-token blocks packed along the token axis, dimensions in the interleaved order
  (j mod 16) * (d/16) + j // 16), ``k4_scale / v4_scale [num_pages, H_kv, b]`` float16. With
  ``int4_frac > 0`` that share of the bf16 pages becomes INT4 pages holding random codes in
  [-7, 7] and random half scales in [0.25, 0.6); otherwise the INT4 pools are poison only.
* ``block_tables [B, max_pages]`` int32 (unused entries -1), ``n_pages [B]`` allocated pages,
  ``context_lens [B]`` cached tokens, ``positions [B]`` 0-based position of the current token.
* page pool: ``refcount [num_pages]`` and a LIFO ``free_stack [num_pages]`` with ``free_top [1]``.
* query-state pool ``[M, 2, H_q, d]`` fp32 (GrowPage App. E.1, Eq. 11, one layer).

Draw order (fixed), with c = ``WORKLOAD_SEED[name]``: metadata from
``numpy.random.Generator(PCG64(1000 + c))``; bulk tensors
from ``torch.Generator(device).manual_seed(1000 + c)`` in the order q, q_hist, K, V, K8, V8 and,
with ``int4_frac > 0``, K4, V4, K4 scales, V4 scales; the INT4 page choice comes from its own
``numpy.random.Generator(PCG64(1000 + c + 7919))`` so that the other draws do not move.
Slots that hold no live token (free pages, the unused tail of a last page, released pages,
the inactive precision of a mixed page) are filled with NaN so that any stray read shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

DTYPE_F32 = "f32"
DTYPE_BF16 = "bf16"

TAG_RELEASE, TAG_FP8, TAG_BF16, TAG_INT4 = 0, 1, 2, 3

WORKLOAD_NAMES = ("tiny", "qwen3_8b", "long_reasoning_d64", "long_reasoning_d128", "prefix_shared",
                  "mixed_precision")
# seed number c of each workload (its draws come from SEED_BASE + c; the two long-reasoning head
# shapes share one)
WORKLOAD_SEED = {"tiny": 1, "qwen3_8b": 2, "long_reasoning_d64": 3, "long_reasoning_d128": 3,
                 "prefix_shared": 4, "mixed_precision": 5}
SEED_BASE = 1000
NUM_SLOTS = 512          # max_num_seqs of the query-state pool (GrowPage App. E.1)
PAST_QUERIES = 32


@dataclasses.dataclass
class Workload:
    name: str
    scale: str
    B: int
    H_q: int
    H_kv: int
    d: int
    page_size: int
    dtype: str
    mixed: bool
    num_pages: int
    max_pages: int
    # tensors
    q: torch.Tensor
    q_hist: torch.Tensor
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    block_tables: torch.Tensor
    n_pages: torch.Tensor
    context_lens: torch.Tensor
    positions: torch.Tensor
    slot_ids: torch.Tensor
    refcount: torch.Tensor
    free_stack: torch.Tensor
    free_top: torch.Tensor
    qstate: torch.Tensor
    # boundary requests and their intended policy (0 auto, 1 force compress, 2 force grow)
    req_idx: torch.Tensor
    req_policy: List[int]
    # mixed-precision extras
    k8: Optional[torch.Tensor] = None
    v8: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    v_scale: Optional[torch.Tensor] = None
    page_tag: Optional[torch.Tensor] = None
    k4: Optional[torch.Tensor] = None
    v4: Optional[torch.Tensor] = None
    k4_scale: Optional[torch.Tensor] = None
    v4_scale: Optional[torch.Tensor] = None
    # method parameters for this workload
    beta_s: float = 0.9
    beta_l: float = 0.999
    p: float = 0.99
    tau: float = 0.0
    k_loc: int = 4
    rope_theta: float = 10000.0
    shared_pages: int = 0
    info: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == DTYPE_F32 else torch.bfloat16

    @property
    def max_context(self) -> int:
        return int(self.info["max_context"])

    def tensor_fields(self):
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, torch.Tensor):
                yield f.name, v

    def to(self, device) -> "Workload":
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Workload(**kw)

    MUTABLE = ("k_pool", "v_pool", "block_tables", "n_pages", "context_lens", "refcount",
               "free_stack", "free_top", "qstate")

    def snapshot(self, names=MUTABLE) -> Dict[str, torch.Tensor]:
        return {n: getattr(self, n).clone() for n in names}

    def restore(self, snap: Dict[str, torch.Tensor]) -> None:
        for n, t in snap.items():
            getattr(self, n).copy_(t)


# --------------------------------------------------------------------------------------------
# per-workload recipes: shapes, dtypes, length mixes and pools of the synthetic workloads
# --------------------------------------------------------------------------------------------

def _spec(name: str, scale: str) -> dict:
    small = scale == "small"
    if name == "tiny":
        return dict(B=2, H_q=8, H_kv=2, d=64, dtype=DTYPE_F32, lens=("fixed", [200, 333]),
                    pool=("fixed", 64), beta_s=0.5, beta_l=0.99, p=0.9, boundary=("all",))
    if name == "qwen3_8b":
        return dict(B=3 if small else 64, H_q=32, H_kv=8, d=128, dtype=DTYPE_BF16,
                    lens=("uniform", 300, 1200) if small else ("uniform", 4096, 16384),
                    pool=("ratio", 1.25), sinks=0.01, boundary=("frac", 1 / 16, 1))
    if name in ("long_reasoning_d64", "long_reasoning_d128"):
        heads = dict(H_q=8, H_kv=2, d=64) if name == "long_reasoning_d64" else dict(H_q=32, H_kv=8, d=128)
        return dict(B=4 if small else 256, dtype=DTYPE_BF16, **heads,
                    lens=("lognormal", 1024, 0.5, 200, 2048) if small
                    else ("lognormal", 8192, 1.0, 512, 32768),
                    pool=("ratio", 1.25), capacity=(0.25, 1.0), boundary=("frac", 1 / 16, 2))
    if name == "prefix_shared":
        return dict(B=4 if small else 128, H_q=40, H_kv=8, d=128, dtype=DTYPE_BF16,
                    shared=64 if small else 2048,
                    lens=("uniform", 100, 400) if small else ("uniform", 1024, 8192),
                    pool=("ratio", 1.25), boundary=("prefix", 1 if small else 8))
    if name == "mixed_precision":
        return dict(B=3 if small else 128, H_q=32, H_kv=8, d=128, dtype=DTYPE_BF16, mixed=True,
                    lens=("uniform", 300, 1200) if small else ("uniform", 8192, 24576),
                    pool=("ratio", 1.25), boundary=("none",))
    raise ValueError(f"unknown workload {name!r}")


def _randn(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _nan_fill_pages(pool: torch.Tensor, pages: np.ndarray) -> None:
    if len(pages):
        idx = torch.as_tensor(pages, dtype=torch.long, device=pool.device)
        pool.index_fill_(0, idx, float("nan"))


def make_workload(name: str, scale: str = "full", device="cpu", seed_offset: int = 0,
                  page_size: int = 16, int4_frac: float = 0.0) -> Workload:
    """Build workload ``name`` (one of WORKLOAD_NAMES) at ``scale`` ("full"/"small").

    ``int4_frac`` (mixed-precision workload only): share of the bf16 pages turned into INT4 pages.
    """
    if name not in WORKLOAD_NAMES:
        raise ValueError(f"unknown workload {name!r}")
    sp = _spec(name, scale)
    seed = SEED_BASE + WORKLOAD_SEED[name] + seed_offset
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    b = page_size
    B, H_q, H_kv, d = sp["B"], sp["H_q"], sp["H_kv"], sp["d"]
    dtype = sp["dtype"]
    tdt = torch.float32 if dtype == DTYPE_F32 else torch.bfloat16
    mixed = bool(sp.get("mixed", False))

    # ---- lengths -----------------------------------------------------------------------
    lens = sp["lens"]
    shared_tokens = int(sp.get("shared", 0))
    if lens[0] == "fixed":
        ctx = np.array(lens[1], dtype=np.int64)
    elif lens[0] == "uniform":
        ctx = rng.integers(lens[1], lens[2], size=B, endpoint=True).astype(np.int64)
    elif lens[0] == "lognormal":
        ell = np.rint(rng.lognormal(math.log(lens[1]), lens[2], size=B))
        ell = np.clip(ell, lens[3], lens[4]).astype(np.int64)
        ctx = ell.copy()
    else:
        raise AssertionError
    logical = ctx.copy()

    # ---- boundary requests -------------------------------------------------------------
    bnd = sp["boundary"]
    req: List[int] = []
    policy: List[int] = []
    capacity = None
    if bnd[0] == "all":
        req = list(range(B))
        policy = [0] * B
    elif bnd[0] == "frac":
        nreq = max(bnd[2], int(round(B * bnd[1]))) if scale == "small" else int(round(B * bnd[1]))
        req = sorted(rng.choice(B, size=nreq, replace=False).tolist())
        policy = [0] * len(req)
    elif bnd[0] == "prefix":
        n_each = bnd[1]
        chosen = rng.choice(B, size=2 * n_each, replace=False).tolist()
        comp, grow = sorted(chosen[:n_each]), sorted(chosen[n_each:])
        req = sorted(comp + grow)
        policy = [1 if r in comp else 2 for r in req]

    if "capacity" in sp:  # per-request retained capacity in pages (long-reasoning mix)
        lo, hi = sp["capacity"]
        u = rng.uniform(lo, hi, size=B)
        capacity = np.maximum(2, np.floor(u * logical / b)).astype(np.int64)
        ctx = np.empty(B, dtype=np.int64)
        for r in range(B):
            P = int(capacity[r])
            if r in req:
                ctx[r] = P * b
            else:
                ctx[r] = rng.integers((P - 1) * b + 1, P * b - 1, endpoint=True)
    elif bnd[0] in ("frac", "prefix"):
        for r in req:  # round the context up to full pages: the request sits at a boundary
            tot = shared_tokens + ctx[r]
            ctx[r] = int(math.ceil(tot / b) * b) - shared_tokens
        logical = ctx.copy()

    # ---- pages and block tables ---------------------------------------------------------
    shared_pages = shared_tokens // b
    if capacity is not None:
        own_pages = capacity.copy()
    else:
        own_pages = np.array([math.ceil((shared_tokens + c) / b) - shared_pages for c in ctx],
                             dtype=np.int64)
    used_pages = int(own_pages.sum()) + shared_pages
    pool = sp["pool"]
    if pool[0] == "fixed":
        num_pages = int(pool[1])
    else:
        unique_tokens = shared_tokens + int(ctx.sum())
        num_pages = max(used_pages + 2, int(math.ceil(pool[1] * unique_tokens / b)))
    perm = rng.permutation(num_pages).astype(np.int64)
    context_lens = (ctx + shared_tokens).astype(np.int64)
    n_pages = (own_pages + shared_pages).astype(np.int64)
    max_pages = int(n_pages.max()) + 4
    bt = np.full((B, max_pages), -1, dtype=np.int64)
    refcount = np.zeros(num_pages, dtype=np.int64)
    cur = 0
    shared_ids = perm[cur:cur + shared_pages]
    cur += shared_pages
    for r in range(B):
        bt[r, :shared_pages] = shared_ids
        k = int(own_pages[r])
        bt[r, shared_pages:shared_pages + k] = perm[cur:cur + k]
        cur += k
    refcount[shared_ids] = B
    for r in range(B):
        for j in range(shared_pages, int(n_pages[r])):
            refcount[bt[r, j]] += 1
    free_ids = perm[cur:]
    free_stack = np.full(num_pages, -1, dtype=np.int64)
    free_stack[:len(free_ids)] = free_ids
    free_top = np.array([len(free_ids)], dtype=np.int64)
    positions = (logical + shared_tokens - 1).astype(np.int64)

    # ---- page tags (mixed precision) -----------------------------------------------------
    page_tag = None
    if mixed:
        n_rel = int(round(0.3 * num_pages))
        n_fp8 = int(round(0.4 * num_pages))
        order = rng.permutation(num_pages)
        page_tag = np.full(num_pages, TAG_BF16, dtype=np.uint8)
        page_tag[order[:n_rel]] = TAG_RELEASE
        page_tag[order[n_rel:n_rel + n_fp8]] = TAG_FP8

    slot_ids = rng.permutation(NUM_SLOTS)[:B].astype(np.int64)

    # ---- bulk tensors ---------------------------------------------------------------------
    q = _randn(gen, (B, H_q, d), device).to(tdt)
    q_hist = _randn(gen, (PAST_QUERIES, B, H_q, d), device).to(tdt)
    k_pool = _randn(gen, (num_pages, H_kv, b, d), device).to(tdt)
    v_pool = _randn(gen, (num_pages, H_kv, b, d), device).to(tdt).transpose(2, 3).contiguous()

    if "sinks" in sp:  # a seeded 1% of each request's tokens get K x 8 (exact in bf16)
        pages, slots = [], []
        for r in range(B):
            n = int(context_lens[r])
            m = int(round(sp["sinks"] * n))
            pos = rng.choice(n, size=m, replace=False)
            pages.append(bt[r, pos // b])
            slots.append(pos % b)
        pg = torch.as_tensor(np.concatenate(pages), device=device)
        sl = torch.as_tensor(np.concatenate(slots), device=device)
        k_pool[pg, :, sl, :] = k_pool[pg, :, sl, :] * 8

    k8 = v8 = k_scale = v_scale = tag_t = None
    if mixed:
        def quant(x):  # x [N, H, b, d] fp32 -> codes, per-row scale
            amax = x.abs().amax(dim=-1)
            scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
            codes = (x / scale[..., None]).to(torch.float8_e4m3fn).view(torch.uint8)
            return codes, scale.to(torch.float32)
        k8, k_scale = quant(_randn(gen, (num_pages, H_kv, b, d), device))
        v8r, v_scale = quant(_randn(gen, (num_pages, H_kv, b, d), device))
        v8 = v8r.transpose(2, 3).contiguous()
        tag_t = torch.as_tensor(page_tag, device=device)
        not_fp8 = np.nonzero(page_tag != TAG_FP8)[0]
        not_bf16 = np.nonzero(page_tag != TAG_BF16)[0]
        _nan_fill_pages(k_pool, not_bf16)
        _nan_fill_pages(v_pool, not_bf16)
        if len(not_fp8):
            idx = torch.as_tensor(not_fp8, device=device)
            k8.index_fill_(0, idx, 0x7F)
            v8.index_fill_(0, idx, 0x7F)
            k_scale.index_fill_(0, idx, float("nan"))
            v_scale.index_fill_(0, idx, float("nan"))

    k4 = v4 = k4_scale = v4_scale = None
    if mixed:
        # INT4 pools: poison (code -8 in both nibbles, NaN scales) except on INT4 pages
        k4 = torch.full((num_pages, H_kv, b, d // 2), 0x88, dtype=torch.uint8, device=device)
        v4 = torch.full((num_pages, H_kv, b // 4, d, 2), 0x88, dtype=torch.uint8, device=device)
        k4_scale = torch.full((num_pages, H_kv, b), float("nan"), dtype=torch.float16, device=device)
        v4_scale = torch.full_like(k4_scale, float("nan"))
        if int4_frac > 0:
            rng4 = np.random.Generator(np.random.PCG64(seed + 7919))
            bf = np.nonzero(page_tag == TAG_BF16)[0]
            pick = np.sort(rng4.permutation(bf)[:int(round(int4_frac * len(bf)))])

            def codes(shape):  # random bytes; a nibble 8 (code -8, outside the range) -> 0
                x = torch.randint(0, 256, shape, generator=gen, device=device, dtype=torch.int32)
                lo, hi = x & 0xF, x >> 4
                lo = torch.where(lo == 8, 0, lo)
                hi = torch.where(hi == 8, 0, hi)
                return (lo | (hi << 4)).to(torch.uint8)

            def scales(shape):
                u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
                return (0.25 + 0.35 * u).to(torch.float16)

            n4 = len(pick)
            idx = torch.as_tensor(pick, dtype=torch.long, device=device)
            k4[idx] = codes((n4, H_kv, b, d // 2))
            v4[idx] = codes((n4, H_kv, b // 4, d, 2))
            k4_scale[idx] = scales((n4, H_kv, b))
            v4_scale[idx] = scales((n4, H_kv, b))
            page_tag[pick] = TAG_INT4
            tag_t = torch.as_tensor(page_tag, device=device)
            _nan_fill_pages(k_pool, pick)
            _nan_fill_pages(v_pool, pick)

    # poison: free pages and the unused tail of every request's last page
    _nan_fill_pages(k_pool, free_ids)
    _nan_fill_pages(v_pool, free_ids)
    if mixed and len(free_ids):
        idx = torch.as_tensor(free_ids, device=device)
        k8.index_fill_(0, idx, 0x7F)
        v8.index_fill_(0, idx, 0x7F)
    for r in range(B):
        n = int(context_lens[r])
        if n % b:
            last = int(bt[r, (n - 1) // b])
            k_pool[last, :, n % b:, :] = float("nan")
            v_pool[last, :, :, n % b:] = float("nan")
            if mixed:
                k8[last, :, n % b:, :] = 0x7F
                v8[last, :, :, n % b:] = 0x7F
                t0 = n % b
                k4[last, :, t0:, :] = 0x88
                k4_scale[last, :, t0:] = float("nan")
                v4_scale[last, :, t0:] = float("nan")
                for t in range(t0, b):  # nibble of token t in its four-token block
                    blk = v4[last, :, t // 4, :, (t % 4) // 2]
                    if t % 2:
                        v4[last, :, t // 4, :, (t % 4) // 2] = (blk & 0x0F) | 0x80
                    else:
                        v4[last, :, t // 4, :, (t % 4) // 2] = (blk & 0xF0) | 0x08

    qstate = torch.full((NUM_SLOTS, 2, H_q, d), float("nan"), dtype=torch.float32, device=device)

    def i32(a):
        return torch.as_tensor(np.asarray(a), dtype=torch.int32, device=device)

    wl = Workload(
        name=name, scale=scale, B=B, H_q=H_q, H_kv=H_kv, d=d, page_size=b, dtype=dtype,
        mixed=mixed, num_pages=num_pages, max_pages=max_pages,
        q=q, q_hist=q_hist, k_pool=k_pool, v_pool=v_pool,
        block_tables=i32(bt), n_pages=i32(n_pages), context_lens=i32(context_lens),
        positions=i32(positions), slot_ids=i32(slot_ids), refcount=i32(refcount),
        free_stack=i32(free_stack), free_top=i32(free_top), qstate=qstate,
        req_idx=i32(req), req_policy=policy,
        k8=k8, v8=v8, k_scale=k_scale, v_scale=v_scale, page_tag=tag_t,
        k4=k4, v4=v4, k4_scale=k4_scale, v4_scale=v4_scale,
        beta_s=sp.get("beta_s", 0.9), beta_l=sp.get("beta_l", 0.999), p=sp.get("p", 0.99),
        tau=0.0, k_loc=max(1, b // 4), rope_theta=10000.0, shared_pages=shared_pages,
        info=dict(max_context=int(context_lens.max()) if B else 0,
                  total_tokens=int(context_lens.sum()), seed=seed,
                  unique_tokens=shared_tokens + int(ctx.sum())),
    )
    return wl


def make_decode_case(B: int, H_q: int, H_kv: int, d: int, page_size: int, lens, dtype: str = DTYPE_BF16,
                     seed: int = 7, device="cpu", boundary=()) -> Workload:
    """A decode batch of arbitrary shape for edge-case tests: the given context lengths, block
    tables drawn as a seeded permutation of a pool 1.25x the pages needed (plus 8 spare), N(0,1)
    q/K/V rounded to `dtype`, NaN in every slot that holds no live token. `boundary` lists request
    indices to mark as boundary requests (summaries initialised from 4 past queries)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    b = page_size
    tdt = torch.float32 if dtype == DTYPE_F32 else torch.bfloat16
    ctx = np.asarray(lens, dtype=np.int64)
    n_pages = np.maximum(1, -(-ctx // b))
    used = int(n_pages.sum())
    num_pages = used + max(8, int(0.25 * used))
    perm = rng.permutation(num_pages).astype(np.int64)
    max_pages = int(n_pages.max()) + 2
    bt = np.full((B, max_pages), -1, dtype=np.int64)
    cur = 0
    for r in range(B):
        k = int(n_pages[r])
        bt[r, :k] = perm[cur:cur + k]
        cur += k
    free_ids = perm[cur:]
    refcount = np.zeros(num_pages, dtype=np.int64)
    refcount[perm[:cur]] = 1
    free_stack = np.full(num_pages, -1, dtype=np.int64)
    free_stack[:len(free_ids)] = free_ids
    q = _randn(gen, (B, H_q, d), device).to(tdt)
    q_hist = _randn(gen, (4, B, H_q, d), device).to(tdt)
    k_pool = _randn(gen, (num_pages, H_kv, b, d), device).to(tdt)
    v_pool = _randn(gen, (num_pages, H_kv, b, d), device).to(tdt).transpose(2, 3).contiguous()
    _nan_fill_pages(k_pool, free_ids)
    _nan_fill_pages(v_pool, free_ids)
    for r in range(B):
        n = int(ctx[r])
        if n % b or n == 0:
            last = int(bt[r, max(0, (n - 1) // b)])
            k_pool[last, :, n % b:, :] = float("nan")
            v_pool[last, :, :, n % b:] = float("nan")
    slot_ids = rng.permutation(max(NUM_SLOTS, B))[:B].astype(np.int64)

    def i32(a):
        return torch.as_tensor(np.asarray(a), dtype=torch.int32, device=device)

    req = sorted(int(r) for r in boundary)
    return Workload(
        name="custom", scale="small", B=B, H_q=H_q, H_kv=H_kv, d=d, page_size=b, dtype=dtype,
        mixed=False, num_pages=num_pages, max_pages=max_pages, q=q, q_hist=q_hist,
        k_pool=k_pool, v_pool=v_pool, block_tables=i32(bt), n_pages=i32(n_pages),
        context_lens=i32(ctx), positions=i32(np.maximum(ctx - 1, 0)), slot_ids=i32(slot_ids),
        refcount=i32(refcount), free_stack=i32(free_stack), free_top=i32([len(free_ids)]),
        qstate=torch.full((max(NUM_SLOTS, B), 2, H_q, d), float("nan"), dtype=torch.float32,
                          device=device),
        req_idx=i32(req), req_policy=[0] * len(req), k_loc=max(1, b // 4),
        info=dict(max_context=int(ctx.max()) if B else 0, total_tokens=int(ctx.sum()), seed=seed,
                  unique_tokens=int(ctx.sum())),
    )


def attach_mixed_pools(wl: Workload, page_tag, seed: int = 0) -> Workload:
    """Turn a bf16 workload into a mixed-precision cache with the given per-page tags: fp8 pages
    get random E4M3 codes of magnitude below 8 and fp32 row scales in [0.01, 0.5), INT4
    pages random code bytes (no nibble 8) and half row scales in [0.01, 0.5); the pools of the
    formats a page does not use, and every pool of a released page, hold poison (NaN bf16,
    NaN fp8 codes, NaN scales, nibble 8). Re-tagging a workload that is already mixed: a page
    that becomes bf16 without having been bf16 holds poison in the bf16 pools, so its K and V
    get fresh standard-normal values (drawn last, so first-time tagging is unchanged)."""
    dev = wl.k_pool.device
    P, H, b, d = wl.k_pool.shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(SEED_BASE + 97 * seed + 5)
    tags = np.asarray(page_tag, dtype=np.uint8)

    def rnd(shape):
        return torch.randint(0, 256, shape, generator=gen, device=dev, dtype=torch.int32)

    def codes8(shape):  # sign, exponent field 0..9 (|value| < 8), mantissa: activation-sized
        x = rnd(shape)
        return ((x & 0x87) | ((x >> 3) % 10 << 3)).to(torch.uint8)

    k8, v8 = codes8((P, H, b, d)), codes8((P, H, d, b))

    def scale(shape, dt):
        u = torch.rand(shape, generator=gen, device=dev, dtype=torch.float32)
        return (0.01 + 0.49 * u).to(dt)

    k_scale, v_scale = scale((P, H, b), torch.float32), scale((P, H, b), torch.float32)

    def codes4(shape):
        x = rnd(shape)
        lo, hi = x & 0xF, x >> 4
        lo = torch.where(lo == 8, 0, lo)
        hi = torch.where(hi == 8, 0, hi)
        return (lo | (hi << 4)).to(torch.uint8)

    k4, v4 = codes4((P, H, b, d // 2)), codes4((P, H, b // 4, d, 2))
    k4_scale, v4_scale = scale((P, H, b), torch.float16), scale((P, H, b), torch.float16)

    def poison(pages, *pools_vals):
        if len(pages):
            idx = torch.as_tensor(pages, dtype=torch.long, device=dev)
            for pool, val in pools_vals:
                pool.index_fill_(0, idx, val)

    old = getattr(wl, "page_tag", None) if getattr(wl, "mixed", False) else None
    if old is not None:
        fresh = np.nonzero((tags == TAG_BF16) & (old.cpu().numpy() != TAG_BF16))[0]
        if len(fresh):
            idx = torch.as_tensor(fresh, dtype=torch.long, device=dev)
            nk = (len(fresh),) + tuple(wl.k_pool.shape[1:])
            nv = (len(fresh),) + tuple(wl.v_pool.shape[1:])
            wl.k_pool.index_copy_(0, idx, _randn(gen, nk, dev).to(wl.k_pool.dtype))
            wl.v_pool.index_copy_(0, idx, _randn(gen, nv, dev).to(wl.v_pool.dtype))
    poison(np.nonzero(tags != TAG_BF16)[0], (wl.k_pool, float("nan")), (wl.v_pool, float("nan")))
    poison(np.nonzero(tags != TAG_FP8)[0], (k8, 0x7F), (v8, 0x7F), (k_scale, float("nan")),
           (v_scale, float("nan")))
    poison(np.nonzero(tags != TAG_INT4)[0], (k4, 0x88), (v4, 0x88), (k4_scale, float("nan")),
           (v4_scale, float("nan")))
    wl.mixed = True
    wl.page_tag = torch.as_tensor(tags, device=dev)
    wl.k8, wl.v8, wl.k_scale, wl.v_scale = k8, v8, k_scale, v_scale
    wl.k4, wl.v4, wl.k4_scale, wl.v4_scale = k4, v4, k4_scale, v4_scale
    return wl
