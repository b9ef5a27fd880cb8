"""Pins for explicit per-pair windows in the oracle.

A stored window table stands in for floor(k * lambda_r); the rule itself is
unchanged: pair r's term of the score is kept while the query-key distance is
at most W_r ("ATFlash — Per-RoPE-Wavelength Attention Windows", README,
"The idea").  Each check compares the oracle with something other than its
own arithmetic: a closed form when every window is 0, a single kept pair
evaluated with complex numbers, brute-force counts, and the derived table.
"""

import numpy as np
import pytest

import oracle
from oracle import window

UNB = 1 << 62


def _inputs(n, d, seed, h_q=2, h_kv=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, h_q, n, d))
    k = rng.standard_normal((1, h_kv, n, d))
    v = rng.standard_normal((1, h_kv, n, d))
    return q, k, v


def test_table_equal_to_derived_reproduces_derived():
    d, base, kt = 64, 1e4, 0.3
    derived = [int(x) for x in window.window_widths(d, base, kt)]
    q, k, v = _inputs(50, d, 1)
    a = oracle.prefill(q, k, v, 0, base, kt)
    b = oracle.prefill(q, k, v, 0, base, 123.0, scaling={"widths": derived})
    assert np.array_equal(a, b)
    assert oracle.pruned_terms(300, 300, 0, d, base, kt) == \
        oracle.pruned_terms(300, 300, 0, d, base, 99.0, scaling={"widths": derived})


def test_all_zero_windows_closed_form():
    """Every window 0: at distance 0 the full score remains and RoPE cancels
    (both sides turn by the same angle), at distance >= 1 every term is
    pruned and the score is 0.  So row n is
    (e^{s q_n.k_n} v_n + sum_{m<n} v_m) / (e^{s q_n.k_n} + n)."""
    d, n = 32, 40
    q, k, v = _inputs(n, d, 2)
    s = 1.0 / np.sqrt(d)
    out = oracle.prefill(q, k, v, 0, 1e4, 1.0, scaling={"widths": [0] * (d // 2)})
    for h in range(2):
        for i in range(n):
            e = np.exp(s * q[0, h, i] @ k[0, 0, i])
            ref = (e * v[0, 0, i] + v[0, 0, :i].sum(axis=0)) / (e + i)
            assert np.allclose(out[0, h, i], ref, rtol=1e-12, atol=1e-12)


def test_single_kept_pair_complex_form():
    """Only pair r keeps its term beyond distance 0.  With the rotate-half
    layout pair r is the complex number x_r + i x_{r+d/2}, turned by
    e^{i p theta_r} at position p, and its term of the score is
    Re(z_q conj(z_k) e^{i (n-m) theta_r})."""
    d, n, base = 16, 30, 100.0
    h = d // 2
    theta = window.pair_frequencies(d, base)
    q, k, v = _inputs(n, d, 3, h_q=1, h_kv=1)
    s = 1.0 / np.sqrt(d)
    for r in (0, 3, h - 1):
        table = [0] * r + [UNB] * (h - r)       # pairs r.. kept everywhere
        if r < h - 1:
            table = [0] * r + [5] + [UNB] * (h - r - 1)   # pair r kept up to distance 5 only
        out = oracle.prefill(q, k, v, 0, base, 1.0, scaling={"widths": table})
        zq = q[0, 0, :, :h] + 1j * q[0, 0, :, h:]
        zk = k[0, 0, :, :h] + 1j * k[0, 0, :, h:]
        for i in range(n):
            sc = np.empty(i + 1)
            for j in range(i + 1):
                delta = i - j
                term = np.real(zq[i] * np.conj(zk[j]) * np.exp(1j * delta * theta))
                keep = np.array([delta <= t for t in table])
                sc[j] = s * term[keep].sum()
            p = np.exp(sc - sc.max())
            ref = (p[:, None] * v[0, 0, :i + 1]).sum(axis=0) / p.sum()
            assert np.allclose(out[0, 0, i], ref, rtol=1e-11, atol=1e-11), (r, i)


def test_counts_closed_form_and_bruteforce():
    d = 16
    h = d // 2
    # every window 0, causal square: every off-diagonal visible cell loses all pairs
    for n in (1, 7, 100):
        pr, tot = oracle.pruned_terms(n, n, 0, d, 1e4, 1.0, scaling={"widths": [0] * h})
        assert tot == h * n * (n + 1) // 2 and pr == h * n * (n - 1) // 2
    rng = np.random.default_rng(11)
    for _ in range(30):
        table = [int(x) for x in np.sort(rng.integers(0, 40, h))]
        n_q, n_kv = int(rng.integers(1, 50)), int(rng.integers(1, 50))
        q0 = int(rng.integers(0, 30))
        causal = bool(rng.integers(0, 2))
        if causal:
            n_kv = min(n_kv, q0 + n_q)
        sc = {"widths": table}
        assert oracle.pruned_terms(n_q, n_kv, q0, d, 1e4, 1.0, causal, True, sc) == \
            oracle.pruned_terms_bruteforce(n_q, n_kv, q0, d, 1e4, 1.0, causal, True, sc)


def test_window_off_and_bad_tables():
    assert list(window.window_widths(8, 1e4, 1.0, False, {"widths": [0, 1, 2, 3]})) == [UNB] * 4
    assert list(window.window_widths(8, 1e4, 1.0, True, {"widths": [0, 1, 2, 1 << 63]})) == [0, 1, 2, UNB]
    with pytest.raises(ValueError):
        window.window_widths(8, 1e4, 1.0, True, {"widths": [0, 1, 2]})
    with pytest.raises(ValueError):
        window.window_widths(8, 1e4, 1.0, True, {"widths": [0, -1, 2, 3]})
