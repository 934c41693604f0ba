"""Pins for the INT4 row quantiser and nibble packing of the oracle (PASK App. B.5)."""
import numpy as np
import pytest
import torch

from oracle import int4
from util import golden_lines


def _golden_cases():
    out = []
    for tok in golden_lines("int4_rows.txt"):
        parts, cur = [], []
        for t in tok:
            if t == ";":
                parts.append(cur)
                cur = []
            else:
                cur.append(t)
        parts.append(cur)
        name, row, scale, codes, packed = parts
        out.append((name[0], [float(x) for x in row], float(scale[0]), [int(c) for c in codes],
                    [int(x, 16) for x in packed]))
    return out


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c[0])
def test_golden_rows(case):
    _, row, scale, codes, packed = case
    c, s = int4.quantize_rows(np.array([row]))
    assert s[0] == scale
    assert c[0].tolist() == codes
    assert int4.pack_pairs(c[0]).tolist() == packed
    back = int4.unpack_pairs(np.array(packed, dtype=np.uint8))
    assert back[:len(codes)].tolist() == codes


def test_scale_rounding_matches_library():
    rng = np.random.default_rng(5)
    # magnitudes from the fp16 subnormal range up to large normals
    amax = np.exp2(rng.uniform(-30, 14, size=4000)) * rng.uniform(1, 2, size=4000)
    rows = np.zeros((amax.size, 3))
    rows[:, 0] = amax
    rows[:, 1] = -amax * rng.uniform(0, 1, size=amax.size)
    _, s = int4.quantize_rows(rows)
    lib = torch.from_numpy(amax / 7.0).to(torch.float16).to(torch.float64).numpy()
    lib = np.maximum(lib, 2.0 ** -24)
    assert np.array_equal(s, lib)


def test_invariants_on_random_rows():
    rng = np.random.default_rng(6)
    rows = np.concatenate([
        rng.standard_normal((300, 128)),
        rng.standard_t(2, size=(300, 128)) * 10,
        rng.standard_normal((100, 64)).repeat(2, axis=1) * 1e-6,
    ])
    c, s = int4.quantize_rows(rows)
    assert c.dtype == np.int8 and np.abs(c).max() <= 7
    assert np.all(np.abs(c).max(axis=1) == 7)                      # the largest element hits 7
    assert np.array_equal(s.astype(np.float16).astype(np.float64), s)  # scales are half values
    ratio = rows / s[:, None]
    inside = np.abs(ratio) <= 7.5
    err = np.abs(rows - c * s[:, None])
    assert np.all(err[inside] <= s[:, None].repeat(rows.shape[1], 1)[inside] / 2)
    assert np.array_equal(c[~inside], np.sign(ratio[~inside]) * 7)   # clipped to +-7
    amax = np.abs(rows).max(axis=1)
    normal = amax / 7 >= 2.0 ** -14                                  # normal half scales
    assert normal[:600].all() and not normal[600:].any()
    assert np.all(np.abs(s - amax / 7)[normal] <= (amax / 7)[normal] * 2.0 ** -11)
    assert np.all(err[normal] <= s[normal, None] / 2)               # no clipping with them
    assert (~inside[600:]).any()                                     # subnormal scales do clip


def test_every_byte_unpacks_like_arithmetic_shifts():
    b = np.arange(256, dtype=np.uint8)
    got = int4.unpack_pairs(b[:, None], axis=-1)                    # [256, 2]
    lo = (b << 4).astype(np.uint8).view(np.int8) >> 4               # sign-extend the low nibble
    hi = b.view(np.int8) >> 4                                       # sign-extend the high nibble
    assert np.array_equal(got[:, 0], lo) and np.array_equal(got[:, 1], hi)
    assert np.array_equal(int4.pack_pairs(got, axis=-1)[:, 0], b)


def test_value_slots_hand_derived():
    """Interleaved dimension order of a value block: dims 16 i + c of one residue c adjacent."""
    slot = int4.value_slot(32)
    assert [slot[j] for j in (0, 16, 1, 17, 2, 15, 31)] == [0, 1, 2, 3, 4, 30, 31]
    slot = int4.value_slot(64)
    assert [slot[j] for j in (0, 16, 32, 48, 1, 63)] == [0, 1, 2, 3, 4, 63]
    assert sorted(int4.value_slot(128).tolist()) == list(range(128))


def test_page_layout_by_brute_force():
    """Keys pack along d, values in four-token blocks; every (token, head) row owns one scale."""
    rng = np.random.default_rng(7)
    H, b, d = 2, 8, 32
    k = rng.standard_normal((H, b, d))
    v = rng.standard_normal((H, d, b)) * 3
    k4, v4, ks, vs = int4.quantize_page_kv(k, v)
    assert k4.shape == (H, b, d // 2) and v4.shape == (H, b // 4, d, 2)
    slot = {j: (j % 16) * (d // 16) + j // 16 for j in range(d)}
    for h in range(H):
        for t in range(b):
            krow, vrow = k[h, t, :], v[h, :, t]
            getters = (
                (krow, ks[h, t], lambda j: (k4[h, t, j // 2] >> 4 * (j % 2)) & 15),
                (vrow, vs[h, t],
                 lambda j: (v4[h, t // 4, slot[j], (t % 4) // 2] >> 4 * (t % 2)) & 15),
            )
            for row, sc, get in getters:
                a = max(abs(x) for x in row)
                s_ref = float(np.float16(a / 7))
                assert sc == s_ref
                for j in range(d):
                    code = int(round(row[j] / s_ref))         # no exact ties in random data
                    code = max(-7, min(7, code))
                    assert int(get(j)) == code & 15
    back = int4.unpack_values(v4)
    assert back.shape == (H, d, b)
    assert np.array_equal(int4.pack_values(back), v4)
