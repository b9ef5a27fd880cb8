"""Pins for the rescaled RoPE frequencies of the oracle (model rope_scaling).

The window tables are built from the RoPE base, the head dim and the model's
rope_scaling ("ATFlash — Per-RoPE-Wavelength Attention Windows", README,
"Using the ports"); the pages name rope_scaling but give no rule, so the
linear rule and the rule of the Llama 3.1 / 3.2 configs are the readings
implemented.  Each check compares the oracle with something other than itself:
a 60-digit mpmath evaluation of the rule, the band structure the rule fixes
exactly, the plain frequencies at factor 1, and brute-force counts.
"""

import math

import mpmath
import numpy as np
import pytest

import oracle
from oracle import window

LLAMA32 = {"rope_type": "llama3", "factor": 32.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
           "original_max_position_embeddings": 8192}
LLAMA31 = {"rope_type": "llama3", "factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
           "original_max_position_embeddings": 8192}
SHAPES = [(128, 5e5, 8.0, LLAMA32), (128, 5e5, 8.0, LLAMA31), (64, 1e6, 8.0, LLAMA31),
          (128, 1e4, 2.0, {"rope_type": "linear", "factor": 4.0}),
          (64, 1e4, 4.0, {"rope_type": "linear", "factor": 2.5})]


def _mp_rule(d, base, sc):
    """The rule written out at 60 digits, pair by pair."""
    mpmath.mp.dps = 60
    out = []
    for r in range(d // 2):
        t = mpmath.power(mpmath.mpf(base), -mpmath.mpf(2 * r) / d)
        if sc["rope_type"] == "linear":
            out.append(t / mpmath.mpf(sc["factor"]))
            continue
        f, a, b = (mpmath.mpf(sc[x]) for x in ("factor", "low_freq_factor", "high_freq_factor"))
        L = mpmath.mpf(sc["original_max_position_embeddings"])
        lam = 2 * mpmath.pi / t
        if lam < L / b:
            out.append(t)
        elif lam > L / a:
            out.append(t / f)
        else:
            s = (L / lam - a) / (b - a)
            out.append((1 - s) * t / f + s * t)
    return out


@pytest.mark.parametrize("d,base,k,sc", SHAPES)
def test_frequencies_and_windows_match_high_precision(d, base, k, sc):
    theta = window.pair_frequencies(d, base, sc)
    ref = _mp_rule(d, base, sc)
    for r in range(d // 2):
        assert abs(theta[r] - float(ref[r])) <= 4e-16 * float(ref[r]), r
    mpmath.mp.dps = 60
    w_ref = [int(mpmath.floor(mpmath.mpf(k) * 2 * mpmath.pi / t)) for t in ref]
    assert list(window.window_widths(d, base, k, True, sc)) == w_ref


@pytest.mark.parametrize("sc", [LLAMA32, LLAMA31])
def test_llama3_band_structure(sc):
    """Short wavelengths keep theta exactly, long ones get exactly theta/f, the
    blend lies strictly between, and the rescaled theta still falls with r."""
    d, base = 128, 5e5
    plain = window.pair_frequencies(d, base)
    scaled = window.pair_frequencies(d, base, sc)
    lam = 2 * math.pi / plain
    L, f = sc["original_max_position_embeddings"], sc["factor"]
    short = lam < L / sc["high_freq_factor"]
    long_ = lam > L / sc["low_freq_factor"]
    mid = ~short & ~long_
    assert short.any() and long_.any() and mid.any()
    assert np.array_equal(scaled[short], plain[short])
    assert np.array_equal(scaled[long_], plain[long_] / f)
    assert np.all(scaled[mid] < plain[mid]) and np.all(scaled[mid] > plain[mid] / f)
    assert np.all(np.diff(scaled) <= 0)


def test_factor_one_is_plain():
    for d, base in ((64, 1e4), (128, 5e5), (128, 1e7)):
        plain = window.pair_frequencies(d, base)
        lin = window.pair_frequencies(d, base, {"rope_type": "linear", "factor": 1.0})
        l3 = window.pair_frequencies(d, base, dict(LLAMA31, factor=1.0))
        assert np.array_equal(lin, plain)
        assert np.allclose(l3, plain, rtol=4e-16, atol=0)
        for k in (1.0, 8.0):
            assert np.array_equal(window.window_widths(d, base, k, True, dict(LLAMA31, factor=1.0)),
                                  window.window_widths(d, base, k, True))


def test_table_equal_to_plain_reproduces_plain():
    d, base = 128, 5e5
    tab = {"rope_type": "table", "theta": list(window.pair_frequencies(d, base))}
    assert np.array_equal(window.window_widths(d, base, 8.0, True, tab), window.window_widths(d, base, 8.0))
    rng = np.random.default_rng(0)
    q = rng.standard_normal((1, 2, 40, d))
    k = rng.standard_normal((1, 1, 40, d))
    v = rng.standard_normal((1, 1, 40, d))
    a = oracle.prefill(q, k, v, 0, base, 0.3)
    b = oracle.prefill(q, k, v, 0, None, 0.3, scaling=tab)
    assert np.array_equal(a, b)


def test_linear_factor_scales_windows():
    """Linear interpolation by f stretches every wavelength by f: W_r equals the
    plain window at k*f."""
    for d, base, k, f in ((64, 1e4, 4.0, 2.0), (128, 5e5, 8.0, 4.0), (128, 1e7, 1.0, 16.0)):
        sc = {"rope_type": "linear", "factor": f}
        got = window.window_widths(d, base, k, True, sc)
        mpmath.mp.dps = 60
        ref = [int(mpmath.floor(mpmath.mpf(k) * f * 2 * mpmath.pi *
                                mpmath.power(mpmath.mpf(base), mpmath.mpf(2 * r) / d))) for r in range(d // 2)]
        assert list(got) == ref


@pytest.mark.parametrize("sc", [LLAMA31, {"rope_type": "linear", "factor": 3.0}])
def test_counts_bruteforce_equals_interval_count(sc):
    rng = np.random.default_rng(7)
    for _ in range(40):
        d = int(rng.choice([8, 16, 64]))
        base = float(rng.choice([20.0, 1e2, 1e4]))
        k = float(rng.choice([0.05, 0.2, 1.0]))
        n_q, n_kv = int(rng.integers(1, 60)), int(rng.integers(1, 60))
        q0 = int(rng.integers(0, 40))
        causal = bool(rng.integers(0, 2))
        if causal:
            n_kv = min(n_kv, q0 + n_q)
        assert oracle.pruned_terms(n_q, n_kv, q0, d, base, k, causal, True, sc) == \
            oracle.pruned_terms_bruteforce(n_q, n_kv, q0, d, base, k, causal, True, sc)


def test_scaled_windows_prune_less_at_long_range():
    """Rescaling only lengthens wavelengths, so no window shrinks and fewer
    terms are pruned at a long context."""
    for sc in (LLAMA32, LLAMA31, {"rope_type": "linear", "factor": 4.0}):
        plain = window.window_widths(128, 5e5, 8.0)
        scaled = window.window_widths(128, 5e5, 8.0, True, sc)
        assert np.all(scaled >= plain)
        p0, t0 = oracle.pruned_terms(131072, 131072, 0, 128, 5e5, 8.0)
        p1, t1 = oracle.pruned_terms(131072, 131072, 0, 128, 5e5, 8.0, scaling=sc)
        assert t0 == t1 and p1 < p0
