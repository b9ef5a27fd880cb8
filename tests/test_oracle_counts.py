"""Pins for oracle.counts.

* brute-force enumeration == per-row interval count == per-pair series for
  the causal square, exactly, over many tiny shapes (including degenerate
  windows, offsets, ragged and non-causal cases);
* the large-N logarithmic approximation agrees with the exact count and grows
  by ln2/ln(base) per doubling of N;
* the shares the pages print (tests/golden/pages_shares.txt).
"""

import math
import os

import numpy as np
import pytest

from oracle import counts, window

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d,base,k", [
    (2, 10.0, 0.5), (4, 100.0, 0.3), (8, 1e4, 0.2), (16, 50.0, 1.0), (16, 1e4, 0.01),
    (6, 3.0, 2.0), (64, 1e4, 4.0), (8, 1e6, math.inf), (12, 7.0, 1e9),
])
def test_bruteforce_equals_interval_count(d, base, k):
    rng = np.random.default_rng(d * 1000 + int(base) % 997)
    for _ in range(12):
        n_q = int(rng.integers(1, 40))
        q_pos0 = int(rng.integers(0, 60))
        n_kv = int(rng.integers(1, 110))
        causal = bool(rng.integers(0, 2))
        on = bool(rng.integers(0, 4))  # mostly on
        a = counts.pruned_terms_bruteforce(n_q, n_kv, q_pos0, d, base, k, causal, on)
        b = counts.pruned_terms(n_q, n_kv, q_pos0, d, base, k, causal, on)
        assert a == b, (n_q, n_kv, q_pos0, causal, on)


@pytest.mark.parametrize("n", [1, 2, 5, 17, 64, 100])
@pytest.mark.parametrize("d,base,k", [(2, 10.0, 0.5), (8, 1e4, 0.2), (16, 50.0, 1.0), (32, 1e3, 0.05)])
def test_square_series_equals_bruteforce(n, d, base, k):
    assert counts.pruned_terms_square_closed_form(n, d, base, k) == \
        counts.pruned_terms_bruteforce(n, n, 0, d, base, k, True, True)


def test_degenerate_counts():
    # every window 0: every off-diagonal term is pruned
    d, n = 8, 30
    w = window.window_widths(d, 1e4, 1e-6, True)
    assert np.all(w == 0)
    p, t = counts.pruned_terms(n, n, 0, d, 1e4, 1e-6)
    assert t == (d // 2) * n * (n + 1) // 2
    assert p == (d // 2) * n * (n - 1) // 2
    # window off: nothing pruned
    assert counts.pruned_terms(n, n, 0, d, 1e4, 4.0, True, False) == (0, t)
    # empty shapes
    assert counts.pruned_terms(0, 10, 0, d, 1e4, 4.0) == (0, 0)
    assert counts.pruned_terms(10, 0, 0, d, 1e4, 4.0) == (0, 0)


def test_chunks_add_up():
    # counts of consecutive query chunks against the growing prefix add up to
    # the one-shot square (the whole-request workload splits prefill this way)
    d, base, k, n, c = 32, 1e4, 0.6, 300, 64
    total_p = total_t = 0
    for s in range(0, n, c):
        e = min(n, s + c)
        p, t = counts.pruned_terms(e - s, e, s, d, base, k)
        total_p += p
        total_t += t
    assert (total_p, total_t) == counts.pruned_terms_square_closed_form(n, d, base, k)


def test_decode_row_count_is_row_of_square():
    d, base, k, n = 64, 1e4, 4.0, 500
    full_p, _ = counts.pruned_terms(n, n, 0, d, base, k)
    upto_p, _ = counts.pruned_terms(n - 1, n - 1, 0, d, base, k)
    row_p, row_t = counts.pruned_terms(1, n, n - 1, d, base, k)
    assert full_p - upto_p == row_p
    assert row_t == (d // 2) * n


@pytest.mark.parametrize("d,base,k,n", [(64, 1e6, 8.0, 32768), (128, 5e5, 8.0, 131072),
                                        (128, 1e7, 64.0, 1048576), (128, 1e7, 8.0, 524288)])
def test_log_approximation_close_to_exact(d, base, k, n):
    p, t = counts.pruned_terms_square_closed_form(n, d, base, k)
    assert abs(p / t - counts.pruned_share_log_approx(n, d, base, k)) < 5e-4


def test_log_growth_per_doubling():
    d, base, k = 64, 1e6, 8.0
    shares = []
    for n in [8192, 16384, 32768, 65536, 131072]:
        p, t = counts.pruned_terms_square_closed_form(n, d, base, k)
        shares.append(p / t)
    steps = np.diff(shares)
    assert np.allclose(steps, math.log(2) / math.log(base), atol=1e-3)


def test_shares_printed_on_pages():
    rows = []
    with open(os.path.join(GOLDEN, "pages_shares.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, d, base, n, k, pct = line.split()[:6]
            rows.append((name, int(d), float(base), int(n), float(k), int(pct)))
    assert len(rows) == 3
    for name, d, base, n, k, pct in rows:
        p, t = counts.pruned_terms_square_closed_form(n, d, base, k)
        assert round(100 * p / t) == pct, name


def test_config_counts_exact_consistency():
    # one-shot square via the per-row route equals the per-pair series at a
    # workload size (per row route is the one used for arbitrary shapes)
    for d, base, k, n in [(64, 1e4, 4.0, 1024), (64, 1e6, 8.0, 32768)]:
        assert counts.pruned_terms(n, n, 0, d, base, k) == \
            counts.pruned_terms_square_closed_form(n, d, base, k)
