"""Pins for oracle.window: integer windows, first retained pair, tile plans.

Each check compares the oracle with something other than itself: a 60-digit
mpmath evaluation of floor(k * 2*pi * base**(2r/d)), the ordering the
definition implies, and a tile plan derived independently from the extreme
distances of each tile.
"""

import math

import mpmath
import numpy as np
import pytest

from oracle import window

CONFIG_SHAPES = [
    # (head_dim, rope_base, k): the five workload shapes
    (64, 1e4, 4.0),
    (64, 1e6, 8.0),
    (128, 5e5, 8.0),
    (128, 1e7, 8.0),
    (128, 1e7, 64.0),
]


def _mp_widths(d, base, k):
    mpmath.mp.dps = 60
    out = []
    for r in range(d // 2):
        w = mpmath.mpf(k) * 2 * mpmath.pi * mpmath.power(mpmath.mpf(base), mpmath.mpf(2 * r) / d)
        out.append(int(mpmath.floor(w)))
    return out


@pytest.mark.parametrize("d,base,k", CONFIG_SHAPES)
def test_widths_match_high_precision(d, base, k):
    got = window.window_widths(d, base, k, True)
    assert got.dtype == np.int64
    assert list(got) == _mp_widths(d, base, k)


def test_widths_match_high_precision_random_grid():
    rng = np.random.default_rng(7)
    for _ in range(40):
        d = int(rng.choice([2, 4, 8, 16, 32, 64, 96, 128, 256]))
        base = float(10 ** rng.uniform(2, 8))
        k = float(rng.choice([0.01, 0.5, 1, 2, 3.5, 4, 8, 64, 1000]))
        assert list(window.window_widths(d, base, k, True)) == _mp_widths(d, base, k)


def test_widths_margin_from_integers_at_configs():
    # fp64 evaluation is safe when w_r is not within ~1e-9 of an integer.
    mpmath.mp.dps = 60
    for d, base, k in CONFIG_SHAPES:
        for r in range(d // 2):
            w = mpmath.mpf(k) * 2 * mpmath.pi * mpmath.power(mpmath.mpf(base), mpmath.mpf(2 * r) / d)
            frac = w - mpmath.floor(w)
            assert min(frac, 1 - frac) > 1e-3


def test_widths_ordering_and_off():
    for d, base, k in CONFIG_SHAPES:
        w = window.window_widths(d, base, k, True)
        assert np.all(np.diff(w) >= 0)            # high frequency = small r = short window
        assert w[-1] > 10 ** 5                    # the lowest-frequency pair reaches far
        off = window.window_widths(d, base, k, False)
        assert np.all(off == window.UNBOUNDED)
        inf = window.window_widths(d, base, math.inf, True)
        assert np.all(inf == window.UNBOUNDED)


def test_first_pair_frequency_is_one():
    # theta_0 = base**0 = 1 for every base, so W_0 = floor(2*pi*k).
    for k in [0.5, 1.0, 4.0, 8.0, 64.0]:
        w = window.window_widths(64, 1e4, k, True)
        assert w[0] == math.floor(2 * math.pi * k)


def test_first_retained_pair_scalar_loop():
    w = window.window_widths(16, 1e4, 1.0, True)
    deltas = np.arange(0, 20000, 37)
    got = window.first_retained_pair(deltas, w)
    for dlt, g in zip(deltas, got):
        cnt = 0
        for r in range(8):
            if w[r] < dlt:
                cnt += 1
        assert g == cnt
    assert window.first_retained_pair(0, w) == 0      # the diagonal keeps every pair


def _plan_from_extremes(n_q, n_kv, q_pos0, causal, tq, tk, w):
    """Independent route: extreme distances of each tile's visible cells in
    closed form, then count windows below them."""
    n_qt, n_kt = -(-n_q // tq), -(-n_kv // tk)
    plan = np.full((n_qt, n_kt, 2), -1, dtype=np.int32)
    for a in range(n_qt):
        n_lo = q_pos0 + a * tq
        n_hi = q_pos0 + min((a + 1) * tq, n_q) - 1
        for b in range(n_kt):
            m_lo = b * tk
            m_hi = min((b + 1) * tk, n_kv) - 1
            if causal:
                if m_lo > n_hi:
                    continue
                dmin = max(0, n_lo - m_hi)
                dmax = n_hi - m_lo
            else:
                if m_hi < n_lo:
                    dmin = n_lo - m_hi
                elif m_lo > n_hi:
                    dmin = m_lo - n_hi
                else:
                    dmin = 0
                dmax = max(abs(n_hi - m_lo), abs(n_lo - m_hi))
            plan[a, b, 0] = int((w < dmin).sum())
            plan[a, b, 1] = int((w < dmax).sum())
    return plan


@pytest.mark.parametrize("n_q,n_kv,q_pos0,causal,tq,tk", [
    (70, 70, 0, True, 16, 8),
    (33, 97, 64, True, 8, 16),
    (50, 41, 0, False, 16, 16),
    (20, 300, 280, True, 4, 32),
    (64, 64, 0, True, 64, 64),
])
def test_tile_plan_matches_extremes(n_q, n_kv, q_pos0, causal, tq, tk):
    w = window.window_widths(16, 100.0, 0.7, True)
    brute = window.tile_plan(n_q, n_kv, q_pos0, causal, tq, tk, w)
    ref = _plan_from_extremes(n_q, n_kv, q_pos0, causal, tq, tk, w)
    np.testing.assert_array_equal(brute, ref)
    assert np.all(brute[..., 0] <= brute[..., 1])


@pytest.mark.parametrize("d,base", [(64, 1e4), (128, 5e5), (128, 1e7)])
def test_pair_wavelengths_definition(d, base):
    # lambda_r is the number of positions in one full turn of pair r
    # ("ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The idea"):
    # pair 0 turns by 1 radian per position, so lambda_0 = 2*pi exactly; a
    # shift by lambda_r turns pair r by exactly 2*pi; consecutive pairs'
    # wavelengths grow by the factor base^(2/d) (60-digit mpmath values)
    lam = window.pair_wavelengths(d, base)
    theta = window.pair_frequencies(d, base)
    assert lam.shape == (d // 2,)
    assert lam[0] == 2 * math.pi
    np.testing.assert_allclose(lam * theta, 2 * math.pi, rtol=1e-15)
    mpmath.mp.dps = 60
    for r in range(d // 2):
        ref = 2 * mpmath.pi * mpmath.power(mpmath.mpf(base), mpmath.mpf(2 * r) / d)
        assert abs(lam[r] - float(ref)) <= 4e-16 * float(ref)
    np.testing.assert_allclose(lam[1:] / lam[:-1], base ** (2.0 / d), rtol=1e-13)


def test_visible_cells_by_hand():
    # queries at positions 1 and 2 (q_pos0 = 1), keys 0..2
    vis, dist = window.visible_cells(2, 3, 1, True)
    assert vis.tolist() == [[True, True, False], [True, True, True]]
    assert dist[vis].tolist() == [1, 0, 2, 1, 0]
    # non-causal: every cell visible, distance |n - m|
    vis, dist = window.visible_cells(2, 3, 1, False)
    assert vis.all()
    assert dist.tolist() == [[1, 0, 1], [2, 1, 0]]
    # queries past the keys (q_pos0 > n_kv): all keys visible
    vis, dist = window.visible_cells(1, 4, 10, True)
    assert vis.all() and dist.tolist() == [[10, 9, 8, 7]]
