"""Symmetric per-row INT4 quantisation of KV rows (PASK App. B.5), float64.

TEST INFRASTRUCTURE ONLY (see the package header): the library never imports this module.

Definition (PASK App. B.5, "Packed attention and quantization"): every K or V row of one
token and one KV head gets its own scale s = fp16(amax / 7), where amax is the largest
magnitude in the row and fp16(.) rounds to the nearest IEEE half value (ties to even); s is
raised to the smallest positive half value (2^-24, a subnormal) when the rounding gives
less. The code of element x is round(x / s) (nearest integer, ties to even) clipped to
[-7, 7], and x is recovered as code * s. A row that is all zeros gets zero codes and scale 1.
Two signed 4-bit codes (two's complement nibbles) share one byte: the element with the even
index along the packing axis sits in the low nibble, the next one in the high nibble.

Storage layout of this library (the scale belongs to the (token, KV head) row in both pools):
* keys pack along the head dimension: a key row of d elements is d/2 bytes, in page order;
* values pack along the token axis in blocks of four tokens: for tokens 4Q .. 4Q+3 and one
  dimension j, byte 0 holds tokens 4Q and 4Q+1 and byte 1 tokens 4Q+2 and 4Q+3, and the d
  two-byte groups of the block are stored in the interleaved dimension order
  slot(j) = (j mod 16) * (d / 16) + floor(j / 16), so that the d/16 dimensions j = 16 i + c
  (i = 0 .. d/16 - 1) of one residue c sit next to each other. A page of one KV head is the
  array [b/4, d, 2] of bytes.

Pinned by: hand-derived rows with their scales, codes and bytes (tests/golden/int4_rows.txt),
including ties in the scale rounding, ties in the code rounding, a subnormal scale, a
subnormal scale that rounds down far enough to clip, the 2^-24 floor and a zero row; the scale
rounding checked against torch's float64 -> float16 conversion on random magnitudes;
invariants (|code| <= 7, a nonzero row reaches 7, with a normal scale every element within
s/2 of code * s, elements beyond 7.5 s clipped to +-7); all 256 byte values unpacked against
arithmetic shifts of int8 and packed back; a page packed into the key rows and the value blocks
by brute force, byte by byte.
"""
import numpy as np

FP16_MIN_POSITIVE = 2.0 ** -24
CODE_MAX = 7


def fp16_round(x) -> np.ndarray:
    """Round float64 values to the nearest IEEE half value (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def quantize_rows(x):
    """Quantise the rows (last axis) of float64 x.

    Returns (codes int8 [..., n], scales float64 [...] holding half values).
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=-1)
    zero = amax == 0
    s = np.maximum(fp16_round(amax / CODE_MAX), FP16_MIN_POSITIVE)
    s = np.where(zero, 1.0, s)
    codes = np.clip(np.rint(x / s[..., None]), -CODE_MAX, CODE_MAX)
    codes = np.where(zero[..., None], 0.0, codes)
    return codes.astype(np.int8), s


def dequantize(codes, scales, axis=-1):
    """code * scale, the scale broadcast along `axis` (the row axis of the codes)."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.expand_dims(np.asarray(scales, dtype=np.float64), axis)
    return c * s


def pack_pairs(codes, axis=-1) -> np.ndarray:
    """Pack signed codes in [-8, 7] two per byte along `axis` (even index in the low nibble)."""
    c = np.moveaxis(np.asarray(codes, dtype=np.int64), axis, -1)
    n = c.shape[-1]
    if n % 2:
        c = np.concatenate([c, np.zeros(c.shape[:-1] + (1,), dtype=np.int64)], axis=-1)
    lo, hi = c[..., 0::2] & 0xF, c[..., 1::2] & 0xF
    return np.moveaxis((lo | (hi << 4)).astype(np.uint8), -1, axis)


def unpack_pairs(packed, axis=-1) -> np.ndarray:
    """Inverse of pack_pairs: signed int8 codes, twice as many along `axis`."""
    p = np.moveaxis(np.asarray(packed, dtype=np.uint8).astype(np.int64), axis, -1)
    lo, hi = p & 0xF, p >> 4
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return np.moveaxis(out.astype(np.int8), -1, axis)


def value_slot(d):
    """Storage slot of each dimension inside a four-token value block."""
    j = np.arange(d)
    return (j % 16) * (d // 16) + j // 16


def pack_values(codes):
    """Value codes [..., d, b] (dimension rows over b tokens) -> bytes [..., b/4, d, 2]."""
    c = np.asarray(codes, dtype=np.int64)
    d, b = c.shape[-2], c.shape[-1]
    pairs = pack_pairs(c, axis=-1)                              # [..., d, b/2], tokens (2i, 2i+1)
    blocks = pairs.reshape(c.shape[:-2] + (d, b // 4, 2))       # [..., d, Q, k]
    blocks = np.moveaxis(blocks, -3, -2)                        # [..., Q, d, k]
    out = np.empty_like(blocks)
    out[..., value_slot(d), :] = blocks
    return out


def unpack_values(packed):
    """Inverse of pack_values: bytes [..., b/4, d, 2] -> signed codes [..., d, b]."""
    p = np.asarray(packed, dtype=np.uint8)
    d = p.shape[-2]
    blocks = p[..., value_slot(d), :]                           # [..., Q, d, k] natural order
    blocks = np.moveaxis(blocks, -2, -3)                        # [..., d, Q, k]
    pairs = blocks.reshape(blocks.shape[:-2] + (blocks.shape[-2] * 2,))
    return unpack_pairs(pairs, axis=-1)


def quantize_page_kv(k_page, v_page):
    """Quantise one page of keys [H, b, d] and values [H, d, b] (values token-contiguous).

    Returns (k4 [H, b, d/2] uint8, v4 [H, b/4, d, 2] uint8, k_scale [H, b], v_scale [H, b]):
    the row of a value is one token over all d dimensions, so its scale runs over axis 1.
    """
    kc, ks = quantize_rows(k_page)                                # rows along d
    vc, vs = quantize_rows(np.swapaxes(np.asarray(v_page), 1, 2))  # [H, b, d] rows along d
    return pack_pairs(kc, axis=-1), pack_values(np.swapaxes(vc, 1, 2)), ks, vs
