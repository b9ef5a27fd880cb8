"""Windowed causal RoPE attention, written out in float64 (prefill and decode).

Definitions followed:

* "ATFlash — Per-RoPE-Wavelength Attention Windows", README, "The idea": a
  score cell is a d-dimensional dot product computed one 2-D frequency pair at
  a time; RoPE rotates pair r of q by n*theta_r and of k by m*theta_r, so the
  pair's contribution depends only on (n - m)*theta_r; once a pair has turned
  k times over the query-key distance its term is set to zero and the sum over
  the remaining pairs is kept; no key is dropped, the online softmax is
  unchanged.
* Same README, "Porting to something else": loops over query n and key m,
  and inside them the pair loop over r, which starts at the window boundary.
* arXiv abstract: the RoPE score decomposes exactly into a sum over its
  frequency pairs; the window prunes the query-key terms of pair r beyond a
  wavelength-proportional distance.

Readings (pages silent):

* rotate-half pairing: pair r is dims (r, r + d/2); rotation at position p:
  x_r' = x_r cos(p theta_r) - x_{r+h} sin(p theta_r),
  x_{r+h}' = x_{r+h} cos(p theta_r) + x_r sin(p theta_r)
  (i.e. z = x_r + i x_{r+h} is multiplied by exp(i p theta_r));
* score s(n, m) = scale * sum_r [dist <= W_r] T_r(n, m), scale = 1/sqrt(d)
  by default, no renormalisation by the retained share; a cell whose every pair
  is pruned has score 0 and stays in the softmax;
* query i of a prefill call is at position q_pos0 + i, key j at position j;
  causal: key visible iff j <= query position; non-causal: window on |n - m|;
* GQA: query head h reads kv head kv_head_of_q[h], default h // (Hq / Hkv);
* inputs of any float dtype are upcast exactly to float64.
"""

import math

import numpy as np

from .window import pair_frequencies, window_widths


def rope(x, positions, theta):
    """Rotate-half RoPE of x[..., P, d] at integer positions[P] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def pair_terms(q_hat, k_hat):
    """T[m, r] = q'_r k'_r + q'_{r+h} k'_{r+h} for one rotated query q_hat[d]
    against rotated keys k_hat[M, d]."""
    h = q_hat.shape[-1] // 2
    return q_hat[None, :h] * k_hat[:, :h] + q_hat[None, h:] * k_hat[:, h:]


def _row_output(q_hat, q_pos, k_hat, v, k_pos, widths, scale, causal, allowed=None):
    """Output of one query row: windowed scores, softmax, weighted sum of v.
    allowed: optional boolean mask over the keys (a token-level selection);
    keys outside it are out of the softmax, and a row attending no key is 0."""
    if causal:
        vis = k_pos <= q_pos
    else:
        vis = np.ones(k_pos.shape, dtype=bool)
    if allowed is not None:
        vis = vis & allowed
    dist = np.abs(q_pos - k_pos[vis])
    if not vis.any():
        return np.zeros(v.shape[-1], dtype=np.float64)
    t = pair_terms(q_hat, k_hat[vis])
    keep = dist[:, None] <= widths[None, :]
    s = scale * np.where(keep, t, 0.0).sum(axis=1)
    p = np.exp(s - s.max())
    return (p @ v[vis]) / p.sum()


def windowed_scores(q, k, q_positions, k_positions, head_dim, rope_base, k_turns,
                    window_on=True, causal=True, scale=None, scaling=None):
    """Scores s[P, M] of one head for queries q[P, d] at q_positions and keys
    k[M, d] at k_positions; invisible cells are -inf."""
    theta = pair_frequencies(head_dim, rope_base, scaling)
    widths = window_widths(head_dim, rope_base, k_turns, window_on, scaling)
    scale = 1.0 / math.sqrt(head_dim) if scale is None or scale <= 0 else scale
    qp = np.asarray(q_positions, dtype=np.int64)
    kp = np.asarray(k_positions, dtype=np.int64)
    q_hat = rope(q, qp, theta)
    k_hat = rope(k, kp, theta)
    out = np.full((len(qp), len(kp)), -np.inf)
    for i in range(len(qp)):
        if causal:
            vis = kp <= qp[i]
            dist = qp[i] - kp
        else:
            vis = np.ones(len(kp), dtype=bool)
            dist = np.abs(qp[i] - kp)
        t = pair_terms(q_hat[i], k_hat)
        keep = dist[:, None] <= widths[None, :]
        s = scale * np.where(keep, t, 0.0).sum(axis=1)
        out[i, vis] = s[vis]
    return out


def _head_map(h_q, h_kv, kv_head_of_q):
    if kv_head_of_q is None:
        if h_q % h_kv:
            raise ValueError("h_q must be a multiple of h_kv without an explicit head map")
        return [h // (h_q // h_kv) for h in range(h_q)]
    return [int(x) for x in kv_head_of_q]


def prefill(q, k, v, q_pos0, rope_base, k_turns, causal=True, window_on=True, scale=None,
            kv_head_of_q=None, query_rows=None, heads=None, batches=None, scaling=None,
            key_blocks=None, block=64):
    """Windowed attention output for prefill, float64.

    q: [B, Hq, Nq, d]; k, v: [B, Hkv, Nkv, d] (pre-RoPE).  Returns
    [len(batches), len(heads), len(query_rows), d] (defaults: all).

    key_blocks: optional boolean block selection [B, Hq, ceil(Nq/block),
    ceil(Nkv/block)]: query row i attends key j only if key_blocks[b, hq,
    i // block, j // block] (a token-level selection, to which the window
    applies on top: "ATFlash: Per-RoPE-Wavelength Attention Windows for
    Compute/Memory-Efficient LLM Inference", arXiv abstract).  Rows attending
    no key give 0.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    bsz, h_q, n_q, d = q.shape
    h_kv, n_kv = k.shape[1], k.shape[2]
    hmap = _head_map(h_q, h_kv, kv_head_of_q)
    theta = pair_frequencies(d, rope_base, scaling)
    widths = window_widths(d, rope_base, k_turns, window_on, scaling)
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else scale
    rows = np.arange(n_q) if query_rows is None else np.asarray(query_rows, dtype=np.int64)
    heads = list(range(h_q)) if heads is None else list(heads)
    batches = list(range(bsz)) if batches is None else list(batches)
    k_pos = np.arange(n_kv, dtype=np.int64)
    out = np.zeros((len(batches), len(heads), len(rows), d), dtype=np.float64)
    k_hat_cache = {}
    for bi, b in enumerate(batches):
        for hi, hq in enumerate(heads):
            kvh = hmap[hq]
            key = (b, kvh)
            if key not in k_hat_cache:
                k_hat_cache.clear()
                k_hat_cache[key] = rope(k[b, kvh], k_pos, theta)
            k_hat = k_hat_cache[key]
            v64 = np.asarray(v[b, kvh], dtype=np.float64)
            q_pos = q_pos0 + rows
            q_hat = rope(q[b, hq, rows], q_pos, theta)
            for ri in range(len(rows)):
                allowed = None
                if key_blocks is not None:
                    allowed = np.asarray(key_blocks[b, hq, int(rows[ri]) // block])[k_pos // block]
                out[bi, hi, ri] = _row_output(q_hat[ri], int(q_pos[ri]), k_hat, v64, k_pos,
                                              widths, scale, causal, allowed)
    return out


def decode(q, k_cache, v_cache, kv_len, q_pos, rope_base, k_turns, causal=True, window_on=True,
           scale=None, kv_head_of_q=None, heads=None, batches=None, scaling=None, key_blocks=None,
           block=64):
    """Windowed attention output for single-token decode, float64.

    q: [B, Hq, d] (pre-RoPE, query of batch b at position q_pos[b]);
    k_cache, v_cache: [B, Hkv, Lmax, d] pre-RoPE, the first kv_len[b] keys of
    batch b valid, key j at position j.  Returns [len(batches), len(heads), d].
    key_blocks: optional boolean [B, Hkv, n_blocks]: kv head h of sequence b
    attends key j only if key_blocks[b, h, j // block] (a token-level
    selection with the window on top); a head attending no key gives 0.
    """
    q = np.asarray(q)
    bsz, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    hmap = _head_map(h_q, h_kv, kv_head_of_q)
    theta = pair_frequencies(d, rope_base, scaling)
    widths = window_widths(d, rope_base, k_turns, window_on, scaling)
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else scale
    heads = list(range(h_q)) if heads is None else list(heads)
    batches = list(range(bsz)) if batches is None else list(batches)
    out = np.zeros((len(batches), len(heads), d), dtype=np.float64)
    for bi, b in enumerate(batches):
        n_kv = int(kv_len[b])
        k_pos = np.arange(n_kv, dtype=np.int64)
        by_kv = {}
        for hi, hq in enumerate(heads):
            by_kv.setdefault(hmap[hq], []).append((hi, hq))
        for kvh, members in by_kv.items():
            k_hat = rope(k_cache[b, kvh, :n_kv], k_pos, theta)
            v64 = np.asarray(v_cache[b, kvh, :n_kv], dtype=np.float64)
            allowed = None
            if key_blocks is not None:
                allowed = np.asarray(key_blocks[b, kvh])[k_pos // block]
            for hi, hq in members:
                pos = int(q_pos[b])
                q_hat = rope(q[b, hq][None, :], np.array([pos]), theta)[0]
                out[bi, hi] = _row_output(q_hat, pos, k_hat, v64, k_pos, widths, scale, causal, allowed)
    return out


def decode_multi(q, k_cache, v_cache, kv_len, q_pos, rope_base, k_turns, window_on=True, scale=None,
                 kv_head_of_q=None, heads=None, batches=None, scaling=None):
    """Windowed causal attention of q_len query tokens per sequence, float64.

    q: [B, T, Hq, d] pre-RoPE; token j of batch b sits at position
    q_pos[b] + j and attends, causally, to keys 0 .. q_pos[b] + j of the first
    kv_len[b] keys (key j at position j), each token with the window measured
    from its own position ("The idea": the window depends on the query-key
    distance only).  Returns [len(batches), T, len(heads), d].
    """
    q = np.asarray(q)
    bsz, n_tok, h_q, d = q.shape
    h_kv = k_cache.shape[1]
    hmap = _head_map(h_q, h_kv, kv_head_of_q)
    theta = pair_frequencies(d, rope_base, scaling)
    widths = window_widths(d, rope_base, k_turns, window_on, scaling)
    scale = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else scale
    heads = list(range(h_q)) if heads is None else list(heads)
    batches = list(range(bsz)) if batches is None else list(batches)
    out = np.zeros((len(batches), n_tok, len(heads), d), dtype=np.float64)
    for bi, b in enumerate(batches):
        n_kv = int(kv_len[b])
        k_pos = np.arange(n_kv, dtype=np.int64)
        for hi, hq in enumerate(heads):
            kvh = hmap[hq]
            k_hat = rope(k_cache[b, kvh, :n_kv], k_pos, theta)
            v64 = np.asarray(v_cache[b, kvh, :n_kv], dtype=np.float64)
            for j in range(n_tok):
                pos = int(q_pos[b]) + j
                q_hat = rope(q[b, j, hq][None, :], np.array([pos]), theta)[0]
                out[bi, j, hi] = _row_output(q_hat, pos, k_hat, v64, k_pos, widths, scale, True)
    return out
