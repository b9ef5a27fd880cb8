"""Per-pair frequencies, wavelengths and integer distance windows (float64).

Definitions followed ("ATFlash — Per-RoPE-Wavelength Attention Windows",
README, section "The idea"; arXiv abstract of the same paper):

* head dim ``d``, ``h = d/2`` rotation pairs; pair ``r`` rotates by the angle
  ``p * theta_r`` at position ``p`` with ``theta_r = base**(-2r/d)``;
* its wavelength is ``lambda_r = 2*pi / theta_r``;
* the window of pair ``r`` is ``w_r = k * lambda_r`` (``k`` = number of full
  turns after which the pair no longer tells positions apart); the pair's term
  of a query-key score is kept while the query-key distance is at most
  ``w_r`` and set to zero beyond it.

Readings (the pages leave these open):

* distances are integers, so ``delta <= w_r`` is the same as
  ``delta <= floor(w_r)``; the integer window ``W_r = floor(w_r)`` is what is
  tabulated here;
* window off, or ``k = +inf``, means every term is kept: ``W_r = UNBOUNDED``;
* ``W_r`` is clamped to ``UNBOUNDED = 2**62`` so it stays an int64.

Rescaled frequencies ("Using the ports": the window tables are built from the
RoPE base, the head dim and the model's rope_scaling; the pages name
rope_scaling but do not define any rule).  Reading: the rotation and the
windows both use the model's rescaled theta_r, and a ``scaling`` dict gives
the rule in the style of a model config:

* ``{"rope_type": "linear", "factor": f}``: every theta_r divided by f;
* ``{"rope_type": "llama3", "factor": f, "low_freq_factor": a,
  "high_freq_factor": b, "original_max_position_embeddings": L}``: the rule of
  the Llama 3.1 / 3.2 configs -- with the plain wavelength lambda_r, a pair
  keeps theta_r when lambda_r < L/b, gets theta_r/f when lambda_r > L/a, and in
  between the blend (1 - s) theta_r/f + s theta_r, s = (L/lambda_r - a)/(b - a);
* ``{"rope_type": "table", "theta": [...]}``: theta_r given per pair.

Any of these may also carry ``"widths": [W_0, ...]``: integer windows given
per pair that stand in for floor(k * lambda_r) (k is then unused); a dict
with only ``"widths"`` keeps the plain frequencies.  The pages build the
windows from the model config; a stored table is this library's extension,
read as "pair r is kept iff the distance is at most the given W_r".

"Porting to something else" asks for the retained prefix per key tile; here a
tile plan gives, per (query tile, key tile), the first pair needed by some
visible cell (``r_any``) and the first pair needed by every visible cell
(``r_full``); pairs below ``r_any`` are never needed in that tile.
"""

import math

import numpy as np

UNBOUNDED = 1 << 62


def pair_frequencies(head_dim, rope_base, scaling=None):
    """theta_r = base**(-2r/d) for r = 0..d/2-1, float64 ("The idea"),
    rescaled by the model's rope scaling rule when ``scaling`` is given."""
    if head_dim <= 0 or head_dim % 2:
        raise ValueError("head_dim must be a positive even integer")
    h = head_dim // 2
    if scaling is not None and scaling.get("rope_type", scaling.get("type")) == "table":
        theta = np.array([float(x) for x in scaling["theta"]], dtype=np.float64)
        if theta.shape != (h,):
            raise ValueError("a frequency table needs head_dim/2 entries")
        return theta
    r = np.arange(h, dtype=np.float64)
    theta = np.power(np.float64(rope_base), -2.0 * r / head_dim)
    kind = None if scaling is None else scaling.get("rope_type", scaling.get("type"))
    if kind is None or kind == "default":
        return theta
    if kind == "linear":
        return theta / np.float64(scaling["factor"])
    if kind == "llama3":
        f = float(scaling["factor"])
        a = float(scaling["low_freq_factor"])
        b = float(scaling["high_freq_factor"])
        L = float(scaling.get("original_max_position_embeddings", scaling.get("original_max_position")))
        out = np.empty(h, dtype=np.float64)
        for i in range(h):
            t = float(theta[i])
            lam = 2.0 * math.pi / t           # plain wavelength of the pair
            if lam < L / b:                   # short wavelengths: unchanged
                out[i] = t
            elif lam > L / a:                 # long wavelengths: interpolated by f
                out[i] = t / f
            else:                             # in between: blend of the two
                s_ = (L / lam - a) / (b - a)
                out[i] = (1.0 - s_) * t / f + s_ * t
        return out
    raise ValueError(f"unknown rope scaling type {kind!r}")


def pair_wavelengths(head_dim, rope_base, scaling=None):
    """lambda_r = 2*pi / theta_r: positions per full turn of pair r."""
    return (2.0 * math.pi) / pair_frequencies(head_dim, rope_base, scaling)


def window_widths(head_dim, rope_base, k_turns, window_on=True, scaling=None):
    """Integer windows W_r = floor(k * lambda_r) as int64 (UNBOUNDED when off;
    the explicit table when ``scaling`` holds "widths").

    Pair r's term is kept at integer distance delta iff delta <= W_r.
    """
    h = head_dim // 2
    if not window_on:
        return np.full(h, UNBOUNDED, dtype=np.int64)
    if scaling is not None and scaling.get("widths") is not None:
        given = [int(x) for x in scaling["widths"]]
        if len(given) != h:
            raise ValueError("an explicit window table needs head_dim/2 entries")
        if min(given) < 0:
            raise ValueError("explicit windows must be >= 0")
        return np.array([min(x, UNBOUNDED) for x in given], dtype=np.int64)
    if math.isinf(k_turns):
        return np.full(h, UNBOUNDED, dtype=np.int64)
    if not k_turns > 0:
        raise ValueError("k_turns must be > 0 when the window is on")
    w = np.float64(k_turns) * pair_wavelengths(head_dim, rope_base, scaling)
    w = np.floor(w)
    out = np.empty(h, dtype=np.int64)
    for r in range(h):
        out[r] = UNBOUNDED if w[r] >= UNBOUNDED else int(w[r])
    return out


def first_retained_pair(delta, widths):
    """r*(delta) = number of pairs whose window is shorter than delta.

    Pairs r with W_r < delta are pruned at that distance; the count of such
    pairs is returned.  Computed by direct comparison against every pair (no
    use of the ordering of W), for scalars or arrays of distances.
    """
    delta = np.asarray(delta, dtype=np.int64)
    w = np.asarray(widths, dtype=np.int64)
    return (w[None, :] < delta.reshape(-1, 1)).sum(axis=1).reshape(delta.shape)


def visible_cells(n_q, n_kv, q_pos0, causal):
    """Boolean [n_q, n_kv] mask of visible (query, key) cells and the distance.

    Query i sits at position q_pos0 + i, key j at position j.  Causal: key j is
    visible iff j <= the query's position; the distance is n - m.  Non-causal:
    every key is visible and the distance is |n - m|.
    """
    n = q_pos0 + np.arange(n_q, dtype=np.int64)[:, None]
    m = np.arange(n_kv, dtype=np.int64)[None, :]
    if causal:
        vis = m <= n
        dist = n - m
    else:
        vis = np.ones((n_q, n_kv), dtype=bool)
        dist = np.abs(n - m)
    return vis, dist


def tile_plan(n_q, n_kv, q_pos0, causal, tile_q, tile_k, widths):
    """Brute-force tile plan: int32 [n_qt, n_kt, 2] of (r_any, r_full).

    For each tile, r*(delta) is evaluated on every visible cell; r_any is its
    minimum (first pair some cell needs) and r_full its maximum (first pair
    every cell needs).  Tiles without a visible cell get (-1, -1).
    """
    vis, dist = visible_cells(n_q, n_kv, q_pos0, causal)
    n_qt = -(-n_q // tile_q)
    n_kt = -(-n_kv // tile_k)
    plan = np.full((n_qt, n_kt, 2), -1, dtype=np.int32)
    for a in range(n_qt):
        for b in range(n_kt):
            sl = (slice(a * tile_q, (a + 1) * tile_q), slice(b * tile_k, (b + 1) * tile_k))
            d = dist[sl][vis[sl]]
            if d.size == 0:
                continue
            rs = first_retained_pair(d, widths)
            plan[a, b, 0] = rs.min()
            plan[a, b, 1] = rs.max()
    return plan
