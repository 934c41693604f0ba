"""OCP FP8 E4M3FN decoding, written from the format definition.

Layout of one byte: sign (1 bit), exponent (4 bits, bias 7), mantissa (3 bits). There are
no infinities; the two patterns S.1111.111 are NaN. Exponent field 0 encodes subnormals
m/8 * 2^(1-7). Largest finite value 448 = 1.75 * 2^8.

Pinned by: every one of the 256 codes against torch's float8_e4m3fn conversion (a library
routine) and hand-derived values in tests/golden/e4m3_codes.txt.
"""
import numpy as np


def e4m3_decode(codes) -> np.ndarray:
    """Return the exact float64 value of each E4M3FN code (uint8 array)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = sign * (m / 8.0) * 2.0 ** (1 - 7)
    out = np.where(e == 0, subnormal, normal)
    out = np.where((e == 0xF) & (m == 0x7), np.nan, out)
    return out
