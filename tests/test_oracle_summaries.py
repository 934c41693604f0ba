"""Pins for the dual-timescale EMA oracle (GrowPage Eq. 6, App. E.1)."""
import numpy as np

from oracle.summaries import update_query_summaries
from util import golden_lines


def _run(qs, beta_s, beta_l, slot=3, M=8):
    T, H, d = qs.shape
    st = np.full((M, 2, H, d), np.nan)
    for t in range(T):
        update_query_summaries(qs[t][None], [slot], [t == 0], st, beta_s, beta_l)
    return st[slot]


def test_golden_sequence():
    rows = {r[0]: [float(x) for x in r[1:]] for r in golden_lines("ema_sequence.txt")}
    bs, bl = rows["beta"]
    st = np.zeros((1, 2, 1, 1))
    for t, qv in enumerate(rows["q"]):
        update_query_summaries(np.array([[[qv]]]), [0], [t == 0], st, bs, bl)
        assert st[0, 0, 0, 0] == rows["short"][t]
        assert st[0, 1, 0, 0] == rows["long"][t]


def test_closed_form():
    rng = np.random.default_rng(0)
    qs = rng.standard_normal((40, 3, 16))
    st = _run(qs, 0.9, 0.999)
    for x, beta in ((0, 0.9), (1, 0.999)):
        n = qs.shape[0]
        ref = beta ** (n - 1) * qs[0] + (1 - beta) * sum(beta ** (n - 1 - k) * qs[k]
                                                          for k in range(1, n))
        assert np.allclose(st[x], ref, rtol=0, atol=1e-12)


def test_beta_zero_is_current_query():
    rng = np.random.default_rng(1)
    qs = rng.standard_normal((10, 2, 8))
    st = _run(qs, 0.0, 0.999)
    assert np.array_equal(st[0], qs[-1])


def test_fresh_overwrites_stale_slot():
    st = np.full((4, 2, 1, 4), 123.0)
    q = np.arange(4.0).reshape(1, 1, 4)
    update_query_summaries(q, [2], [True], st, 0.9, 0.999)
    assert np.array_equal(st[2, 0], q[0]) and np.array_equal(st[2, 1], q[0])
    assert np.all(st[[0, 1, 3]] == 123.0)
    update_query_summaries(q * 0, [2], [False], st, 0.5, 0.75)
    assert np.array_equal(st[2, 0], 0.5 * q[0]) and np.array_equal(st[2, 1], 0.75 * q[0])
