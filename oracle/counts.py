"""Pruned and total pair-term counts of the per-RoPE-wavelength window.

The pages state that the reduction does not depend on the input and has a
closed form that grows logarithmically with the sequence length N, so the cost
is known before running ("ATFlash — Per-RoPE-Wavelength Attention Windows",
README, "The idea"; arXiv abstract).  They print the shares (37-48% within
native context, 57% at 1M) but not the formula.

Unit (reading): one "term" is one (query, key, pair) triple, i.e. the two
products of pair r in one score cell.  Counts are per (batch, query head) over
the visible cells: query i at position q_pos0 + i, key j at position j,
causal (key visible iff j <= query position, distance n - m) or not (every
key visible, distance |n - m|).  A term is pruned iff distance > W_r.

Three routes are given, written independently of each other:

* :func:`pruned_terms_bruteforce` enumerates every visible cell;
* :func:`pruned_terms` counts, row by row and pair by pair, the distances of
  the row's visible range that lie beyond W_r (exact, any shape);
* :func:`pruned_terms_square_closed_form` sums an arithmetic series per pair
  for the full causal N x N square (exact);
* :func:`pruned_share_log_approx` is the large-N continuum approximation of
  the share, the logarithmic closed form the pages speak of (approximate).
"""

import math

import numpy as np

from .window import window_widths, visible_cells


def pruned_terms(n_q, n_kv, q_pos0, head_dim, rope_base, k_turns, causal=True, window_on=True,
                 scaling=None):
    """Exact (pruned, total) pair-term counts; per-row interval counting.

    Row n sees a contiguous set of distances; pair r is pruned on the part of
    it that lies above W_r.  Sums are taken in Python integers (no overflow).
    """
    h = head_dim // 2
    if n_q <= 0 or n_kv <= 0:
        return 0, 0
    widths = window_widths(head_dim, rope_base, k_turns, window_on, scaling)
    n = q_pos0 + np.arange(n_q, dtype=np.int64)
    pruned = 0
    if causal:
        last = np.minimum(n, n_kv - 1)          # last visible key of row n
        d_lo = n - last                         # smallest visible distance
        d_hi = n                                # largest (key 0)
        visible = int((last + 1).sum())
        for r in range(h):
            w = np.int64(widths[r])
            cnt = d_hi - np.maximum(w, d_lo - 1)
            pruned += int(np.clip(cnt, 0, None).sum())
    else:
        visible = n_q * n_kv
        for r in range(h):
            w = np.int64(widths[r])
            below = np.clip(n - w, 0, n_kv)                 # keys m <= n - W - 1
            above = np.clip(n_kv - (n + w + 1), 0, n_kv)    # keys m >= n + W + 1
            pruned += int(below.sum()) + int(above.sum())
    return pruned, h * visible


def pruned_terms_bruteforce(n_q, n_kv, q_pos0, head_dim, rope_base, k_turns, causal=True,
                            window_on=True, scaling=None):
    """Exact counts by enumerating every visible (query, key, pair) triple.

    Only for small sizes (materialises the n_q x n_kv cell grid).
    """
    h = head_dim // 2
    if n_q <= 0 or n_kv <= 0:
        return 0, 0
    widths = window_widths(head_dim, rope_base, k_turns, window_on, scaling)
    vis, dist = visible_cells(n_q, n_kv, q_pos0, causal)
    d = dist[vis]
    pruned = 0
    for r in range(h):
        pruned += int((d > widths[r]).sum())
    return pruned, h * int(vis.sum())


def pruned_terms_square_closed_form(n, head_dim, rope_base, k_turns, window_on=True):
    """Exact counts for the full causal N x N square, one series per pair.

    In an N x N causal square, distance delta occurs N - delta times
    (delta = 0..N-1).  Pair r is pruned at every delta > W_r, so its count is
    sum_{delta=W_r+1}^{N-1} (N - delta) = x(x+1)/2 with x = N - 1 - W_r (0 if
    x <= 0).  Total terms: h * N(N+1)/2.
    """
    h = head_dim // 2
    widths = window_widths(head_dim, rope_base, k_turns, window_on)
    pruned = 0
    for w in widths:
        x = n - 1 - int(w)
        if x > 0:
            pruned += x * (x + 1) // 2
    return pruned, h * n * (n + 1) // 2


def pruned_share_log_approx(n, head_dim, rope_base, k_turns):
    """Large-N share of pruned terms: [ln(N/(2 pi k)) - 3/2]/ln(base) + 1/d.

    Continuum limit of the square count: with u = 2r/d the window is
    2*pi*k*base**u; pairs with window < N (u < u* = ln(N/(2 pi k))/ln base)
    contribute (1 - W/N)**2 of their row share; integrating over u and adding
    the half-weight end term of the sum over r gives the expression.  Valid for
    2*pi*k << N <= the longest window; it grows by ln 2 / ln(base) per doubling
    of N, the logarithmic growth the pages state.
    """
    return (math.log(n / (2.0 * math.pi * k_turns)) - 1.5) / math.log(rope_base) + 1.0 / head_dim


def pruned_terms_blocks(n_q, n_kv, q_pos0, head_dim, rope_base, k_turns, selected, causal=True,
                        window_on=True, scaling=None, block=64):
    """Exact (pruned, total) pair-term counts over the cells a block selection
    attends (one head): selected[qb, kb] (boolean, ceil(n_q/block) x
    ceil(n_kv/block)) lets query rows [qb*block, ...) see keys [kb*block, ...).
    Per row and selected key block, the attended keys form one interval, and
    pair r is pruned on the part of its distances above W_r (interval
    counting in Python integers)."""
    h = head_dim // 2
    if n_q <= 0 or n_kv <= 0:
        return 0, 0
    widths = window_widths(head_dim, rope_base, k_turns, window_on, scaling)
    selected = np.asarray(selected, dtype=bool)
    pruned = 0
    visible = 0
    for i in range(n_q):
        n = q_pos0 + i
        for kb in np.nonzero(selected[i // block])[0]:
            m0 = int(kb) * block
            m1 = min(n_kv, m0 + block) - 1             # keys [m0, m1]
            if causal:
                m1 = min(m1, n)
            if m1 < m0:
                continue
            visible += m1 - m0 + 1
            for r in range(h):
                w = int(widths[r])
                # keys with n - m > w: m <= n - w - 1
                pruned += max(0, min(m1, n - w - 1) - m0 + 1)
                if not causal:
                    # keys with m - n > w: m >= n + w + 1
                    pruned += max(0, m1 - max(m0, n + w + 1) + 1)
    return pruned, h * visible


def pruned_terms_blocks_bruteforce(n_q, n_kv, q_pos0, head_dim, rope_base, k_turns, selected,
                                   causal=True, window_on=True, scaling=None, block=64):
    """Same counts by enumerating every attended (query, key, pair) triple
    (small sizes only: materialises the cell grid)."""
    h = head_dim // 2
    if n_q <= 0 or n_kv <= 0:
        return 0, 0
    widths = window_widths(head_dim, rope_base, k_turns, window_on, scaling)
    vis, dist = visible_cells(n_q, n_kv, q_pos0, causal)
    sel = np.asarray(selected, dtype=bool)
    qb = np.arange(n_q) // block
    kb = np.arange(n_kv) // block
    vis = vis & sel[qb[:, None], kb[None, :]]
    d = dist[vis]
    pruned = 0
    for r in range(h):
        pruned += int((d > widths[r]).sum())
    return pruned, h * int(vis.sum())
