"""Paged decode attention, float64.

Definition (PASK, Sec. 3.1 "KV cache"): for one query q and the cached keys/values of its
KV head, o = V softmax(K^T q / sqrt(d_k)). Keys and values are found through the request's
block table: token slot j lives in physical page bt[j // b] at offset j % b (GrowPage Sec. 4.2:
a page appended to the block table leaves the attention interface unchanged). GQA maps query
head g to KV head g // G (PASK App. B.5). With mixed-precision pages (PASK App. B.2 and B.5)
a released page contributes no tokens, an fp8 page's element is code value * row scale, an
INT4 page's element is its signed nibble times the row's half-precision scale (App. B.5, the
packing described in oracle.int4), and absolute token positions survive the gaps.

Split-KV merge (PASK App. B.5): partial results (v_j, l_j, u_j) = (max logit, sum of
exponentials, unnormalised output) of disjoint token sets combine as
o = sum_j e^{v_j - v} u_j / sum_j e^{v_j - v} l_j with v = max_j v_j.

Pinned by: softmax weights sum to one; a contiguous layout equals any block-table permutation;
equality with torch.nn.functional.scaled_dot_product_attention in float64 on the gathered
tokens; random split partitions merged equal the single pass; a released page equals deleting
its tokens; an INT4 page equals a float page holding its dequantised values; a hand-computed
two-token example (tests/golden/decode_tiny.txt).
"""
import numpy as np

from .fp8 import e4m3_decode
from .int4 import unpack_pairs, unpack_values

TAG_RELEASE, TAG_FP8, TAG_BF16, TAG_INT4 = 0, 1, 2, 3


def gather_request_kv(r, k_pool, v_pool, block_tables, context_lens, page_size,
                      page_tag=None, k8=None, v8=None, k_scale=None, v_scale=None,
                      k4=None, v4=None, k4_scale=None, v4_scale=None):
    """Visible keys and values of request r as float64 arrays [H_kv, n_vis, d].

    k_pool is [num_pages, H_kv, b, d]; v_pool is [num_pages, H_kv, d, b] (token axis last).
    INT4 pools: k4 [num_pages, H_kv, b, d/2] (packed along d), v4 [num_pages, H_kv, b/4, d, 2]
    (four-token blocks packed along tokens, dimensions interleaved as in oracle.int4),
    k4_scale / v4_scale [num_pages, H_kv, b] half values.
    Also returns the absolute slot index of every visible token.
    """
    n = int(context_lens[r])
    b = page_size
    slots = np.arange(n)
    pages = np.asarray(block_tables[r])[slots // b].astype(np.int64)
    offs = slots % b
    if page_tag is not None:
        tags = np.asarray(page_tag)[pages]
        keep = tags != TAG_RELEASE
        slots, pages, offs, tags = slots[keep], pages[keep], offs[keep], tags[keep]
    k = np.asarray(k_pool)[pages, :, offs, :].astype(np.float64)          # [n, H, d]
    v = np.asarray(v_pool)[pages, :, :, offs].astype(np.float64)          # [n, H, d]
    if page_tag is not None:
        f8 = tags == TAG_FP8
        if f8.any():
            kc = e4m3_decode(np.asarray(k8)[pages[f8], :, offs[f8], :])
            vc = e4m3_decode(np.asarray(v8)[pages[f8], :, :, offs[f8]])
            ks = np.asarray(k_scale)[pages[f8], :, offs[f8]].astype(np.float64)
            vs = np.asarray(v_scale)[pages[f8], :, offs[f8]].astype(np.float64)
            k[f8] = kc * ks[..., None]
            v[f8] = vc * vs[..., None]
        i4 = tags == TAG_INT4
        if i4.any():
            pg, of = pages[i4], offs[i4]
            kc = unpack_pairs(np.asarray(k4)[pg, :, of, :], axis=-1)              # [m, H, d]
            vfull = unpack_values(np.asarray(v4)[pg])                             # [m, H, d, b]
            vc = vfull[np.arange(len(pg)), :, :, of]                              # [m, H, d]
            ks = np.asarray(k4_scale)[pg, :, of].astype(np.float64)
            vs = np.asarray(v4_scale)[pg, :, of].astype(np.float64)
            k[i4] = kc.astype(np.float64) * ks[..., None]
            v[i4] = vc.astype(np.float64) * vs[..., None]
    return k.transpose(1, 0, 2), v.transpose(1, 0, 2), slots


def attend(q, k, v, sm_scale):
    """Softmax attention of queries q [G, d] over k, v [n, d]; returns (o [G, d], lse [G]).

    With no visible token the output is zero and the log-sum-exp is -inf.
    """
    G, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((G, d)), np.full(G, -np.inf)
    z = (q @ k.T) * sm_scale
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    s = w.sum(axis=1, keepdims=True)
    o = (w / s) @ v
    lse = (m + np.log(s))[:, 0]
    return o, lse


def paged_decode_attn(q, k_pool, v_pool, block_tables, context_lens, page_size, sm_scale,
                      page_tag=None, k8=None, v8=None, k_scale=None, v_scale=None,
                      k4=None, v4=None, k4_scale=None, v4_scale=None, requests=None):
    """Decode attention for every request (or the listed ones).

    q: [B, H_q, d]. Returns out [B, H_q, d] and lse [B, H_q] in float64; rows of requests not
    listed are NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    B, H_q, d = q.shape
    H_kv = np.asarray(k_pool).shape[1]
    G = H_q // H_kv
    out = np.full((B, H_q, d), np.nan)
    lse = np.full((B, H_q), np.nan)
    for r in (range(B) if requests is None else requests):
        k, v, _ = gather_request_kv(r, k_pool, v_pool, block_tables, context_lens, page_size,
                                    page_tag, k8, v8, k_scale, v_scale, k4, v4, k4_scale,
                                    v4_scale)
        for h in range(H_kv):
            o, l_ = attend(q[r, h * G:(h + 1) * G], k[h], v[h], sm_scale)
            out[r, h * G:(h + 1) * G] = o
            lse[r, h * G:(h + 1) * G] = l_
    return out, lse


def split_partial(q, k, v, sm_scale):
    """Partial (v_j, l_j, u_j) of one token subset: max logit, sum of exponentials and the
    unnormalised output (PASK App. B.5)."""
    z = (q @ k.T) * sm_scale
    vmax = z.max(axis=1)
    e = np.exp(z - vmax[:, None])
    return vmax, e.sum(axis=1), e @ v


def merge_splits(parts):
    """Combine split partials with the PASK App. B.5 rule; returns (o, lse)."""
    vs = np.stack([p[0] for p in parts])            # [S, G]
    ls = np.stack([p[1] for p in parts])            # [S, G]
    us = np.stack([p[2] for p in parts])            # [S, G, d]
    vmax = vs.max(axis=0)
    w = np.exp(vs - vmax)
    num = (w[..., None] * us).sum(axis=0)
    den = (w * ls).sum(axis=0)
    return num / den[:, None], vmax + np.log(den)
