"""Pins for oracle.attention against routes that do not reuse its code.

* RoPE == multiplication of z = x_r + i x_{r+h} by exp(i p theta_r);
* pair term == Re(z_q conj(z_k) exp(i (n-m) theta_r)) on un-rotated inputs
  (the relative-angle property the pages state);
* window off == textbook causal RoPE attention (numpy complex route, and
  torch scaled_dot_product_attention in float64 on the CPU);
* shift invariance of the windowed scores;
* closed forms: every window 0 (only the diagonal keeps its score) and d = 2;
* a pure-Python scalar triple loop on tiny inputs with pruning active;
* consistency across entry points: decode row == prefill row, chunked
  prefill == one-shot, GQA head == single head on its kv head;
* planted mistakes (wrong rotation sign, wrong pair pairing, inclusive/
  exclusive boundary, dropped scale) are caught by these pins.
"""

import cmath
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, window


def _cplx(x):
    h = x.shape[-1] // 2
    return x[..., :h] + 1j * x[..., h:]


def _rope_complex(x, pos, theta):
    z = _cplx(np.asarray(x, dtype=np.float64))
    zr = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :])
    return np.concatenate([zr.real, zr.imag], axis=-1)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rope_is_complex_rotation():
    theta = window.pair_frequencies(64, 1e4)
    x = _rand((50, 64), 1)
    pos = np.arange(1000, 1050)
    np.testing.assert_allclose(attention.rope(x, pos, theta), _rope_complex(x, pos, theta),
                               rtol=0, atol=1e-12)


def test_pair_term_depends_on_relative_angle_only():
    d, base = 16, 1e4
    theta = window.pair_frequencies(d, base)
    q, k = _rand(d, 2), _rand((30, d), 3)
    n, mpos = 777, np.arange(700, 730)
    t = attention.pair_terms(attention.rope(q[None], [n], theta)[0], attention.rope(k, mpos, theta))
    zq, zk = _cplx(q), _cplx(k)
    ref = (zq[None, :] * np.conj(zk) * np.exp(1j * (n - mpos)[:, None] * theta[None, :])).real
    np.testing.assert_allclose(t, ref, atol=1e-12)
    # and the pair terms sum to the plain dot product of the rotated vectors
    qh = attention.rope(q[None], [n], theta)[0]
    kh = attention.rope(k, mpos, theta)
    np.testing.assert_allclose(t.sum(1), kh @ qh, atol=1e-12)


def _textbook(q, k, v, q_pos0, base, scale, causal=True):
    """Plain causal RoPE attention of one head (complex-rotation route)."""
    n_q, d = q.shape
    n_kv = k.shape[0]
    theta = window.pair_frequencies(d, base)
    qh = _rope_complex(q, q_pos0 + np.arange(n_q), theta)
    kh = _rope_complex(k, np.arange(n_kv), theta)
    s = scale * qh @ kh.T
    if causal:
        s = np.where(np.arange(n_kv)[None, :] <= (q_pos0 + np.arange(n_q))[:, None], s, -np.inf)
    s = s - s.max(1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(1, keepdims=True)


@pytest.mark.parametrize("q_pos0,n_q,n_kv,causal", [(0, 40, 40, True), (25, 15, 40, True),
                                                    (0, 20, 33, False)])
def test_window_off_equals_textbook(q_pos0, n_q, n_kv, causal):
    d, base = 32, 1e4
    q, k, v = _rand((1, 1, n_q, d), 4), _rand((1, 1, n_kv, d), 5), _rand((1, 1, n_kv, d), 6)
    out = oracle.prefill(q, k, v, q_pos0, base, 4.0, causal=causal, window_on=False)
    ref = _textbook(q[0, 0], k[0, 0], v[0, 0], q_pos0, base, 1 / math.sqrt(d), causal)
    np.testing.assert_allclose(out[0, 0], ref, atol=1e-12)
    # k = +inf with the window on is the same thing
    out2 = oracle.prefill(q, k, v, q_pos0, base, math.inf, causal=causal, window_on=True)
    assert np.array_equal(out, out2)


def test_window_off_equals_torch_sdpa():
    d, base, n = 64, 1e4, 96
    q, k, v = _rand((1, 2, n, d), 7), _rand((1, 2, n, d), 8), _rand((1, 2, n, d), 9)
    out = oracle.prefill(q, k, v, 0, base, 4.0, window_on=False)
    theta = window.pair_frequencies(d, base)
    qh = torch.tensor(np.stack([_rope_complex(q[0, h], np.arange(n), theta) for h in range(2)]))[None]
    kh = torch.tensor(np.stack([_rope_complex(k[0, h], np.arange(n), theta) for h in range(2)]))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, torch.tensor(v), is_causal=True)
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("shift", [12345, 10 ** 6])
def test_windowed_scores_shift_invariant(shift):
    d, base, k = 32, 1e4, 0.5
    q, kk = _rand((12, d), 10), _rand((40, d), 11)
    qp = np.arange(28, 40)
    kp = np.arange(40)
    a = attention.windowed_scores(q, kk, qp, kp, d, base, k)
    b = attention.windowed_scores(q, kk, qp + shift, kp + shift, d, base, k)
    fin = np.isfinite(a)
    assert np.array_equal(fin, np.isfinite(b))
    np.testing.assert_allclose(a[fin], b[fin], atol=1e-9)


def test_degenerate_window_closed_form():
    # every W_r = 0: all off-diagonal scores are 0, the diagonal keeps the
    # full dot product (RoPE cancels at equal positions).
    d, base, n = 16, 1e4, 30
    k_turns = 1e-6
    assert np.all(window.window_widths(d, base, k_turns) == 0)
    q, k, v = _rand((1, 1, n, d), 12), _rand((1, 1, n, d), 13), _rand((1, 1, n, d), 14)
    out = oracle.prefill(q, k, v, 0, base, k_turns)[0, 0]
    scale = 1 / math.sqrt(d)
    for i in range(n):
        e = math.exp(scale * float(q[0, 0, i] @ k[0, 0, i]))
        ref = (v[0, 0, :i].sum(0) + e * v[0, 0, i]) / (i + e)
        np.testing.assert_allclose(out[i], ref, atol=1e-12)


def test_d2_closed_form():
    # d = 2: theta_0 = 1, s = scale [delta <= W_0] |z_q||z_k| cos(delta + arg z_q - arg z_k)
    base, k_turns, n = 1e4, 2.0, 40
    w0 = math.floor(2 * math.pi * k_turns)
    q, kk = _rand((n, 2), 15), _rand((n, 2), 16)
    s = attention.windowed_scores(q, kk, np.arange(n), np.arange(n), 2, base, k_turns)
    for i in range(n):
        for j in range(i + 1):
            zq, zk = complex(*q[i]), complex(*kk[j])
            dlt = i - j
            ref = 0.0 if dlt > w0 else abs(zq) * abs(zk) * math.cos(dlt + cmath.phase(zq) - cmath.phase(zk))
            assert abs(s[i, j] - ref / math.sqrt(2)) < 1e-12


def _scalar_loops(q, k, v, q_pos0, base, k_turns, causal):
    """Pure-Python triple loop (query, key, pair) of the windowed definition."""
    n_q, d = len(q), len(q[0])
    h = d // 2
    scale = 1 / math.sqrt(d)
    out = []
    for i in range(n_q):
        n = q_pos0 + i
        scores, vals = [], []
        for m in range(len(k)):
            if causal and m > n:
                continue
            dist = abs(n - m)
            s = 0.0
            for r in range(h):
                th = base ** (-2.0 * r / d)
                if dist > math.floor(k_turns * 2 * math.pi / th):
                    continue
                a, b = n * th, m * th
                q1 = q[i][r] * math.cos(a) - q[i][r + h] * math.sin(a)
                q2 = q[i][r + h] * math.cos(a) + q[i][r] * math.sin(a)
                k1 = k[m][r] * math.cos(b) - k[m][r + h] * math.sin(b)
                k2 = k[m][r + h] * math.cos(b) + k[m][r] * math.sin(b)
                s += q1 * k1 + q2 * k2
            scores.append(scale * s)
            vals.append(v[m])
        mx = max(scores)
        ps = [math.exp(s - mx) for s in scores]
        tot = sum(ps)
        out.append([sum(p * vv[c] for p, vv in zip(ps, vals)) / tot for c in range(d)])
    return np.array(out)


@pytest.mark.parametrize("q_pos0,n_q,n_kv,causal", [(0, 9, 9, True), (4, 6, 12, True), (0, 7, 10, False)])
def test_scalar_triple_loop(q_pos0, n_q, n_kv, causal):
    d, base, k_turns = 6, 10.0, 0.3        # windows [1, 4, 8]: pruning is active
    assert list(window.window_widths(d, base, k_turns)) == [1, 4, 8]
    q, k, v = _rand((n_q, d), 17), _rand((n_kv, d), 18), _rand((n_kv, d), 19)
    out = oracle.prefill(q[None, None], k[None, None], v[None, None], q_pos0, base, k_turns,
                         causal=causal)[0, 0]
    ref = _scalar_loops(q.tolist(), k.tolist(), v.tolist(), q_pos0, base, k_turns, causal)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_nothing_pruned_is_window_off_bitwise():
    d, base, n = 32, 1e4, 50
    q, k, v = _rand((1, 1, n, d), 20), _rand((1, 1, n, d), 21), _rand((1, 1, n, d), 22)
    k_turns = 10.0                      # W_0 = 62 >= n - 1
    assert window.window_widths(d, base, k_turns)[0] >= n - 1
    a = oracle.prefill(q, k, v, 0, base, k_turns, window_on=True)
    b = oracle.prefill(q, k, v, 0, base, k_turns, window_on=False)
    assert np.array_equal(a, b)


def test_decode_row_equals_prefill_row():
    d, base, k_turns, n = 32, 1e4, 0.5, 60
    q, k, v = _rand((2, 4, n, d), 23), _rand((2, 2, n, d), 24), _rand((2, 2, n, d), 25)
    pre = oracle.prefill(q, k, v, 0, base, k_turns)
    for row in [0, 17, n - 1]:
        dec = oracle.decode(q[:, :, row], k, v, [row + 1, row + 1], [row, row], base, k_turns)
        np.testing.assert_allclose(dec, pre[:, :, row], atol=1e-12)


def test_chunked_prefill_equals_one_shot():
    d, base, k_turns, n, c = 32, 1e4, 0.5, 70, 16
    q, k, v = _rand((1, 2, n, d), 26), _rand((1, 2, n, d), 27), _rand((1, 2, n, d), 28)
    full = oracle.prefill(q, k, v, 0, base, k_turns)
    for s in range(0, n, c):
        e = min(n, s + c)
        part = oracle.prefill(q[:, :, s:e], k[:, :, :e], v[:, :, :e], s, base, k_turns)
        np.testing.assert_allclose(part, full[:, :, s:e], atol=1e-12)


def test_gqa_head_is_single_head_on_its_kv_head():
    d, base, k_turns, n = 16, 1e4, 0.5, 30
    q, k, v = _rand((1, 6, n, d), 29), _rand((1, 2, n, d), 30), _rand((1, 2, n, d), 31)
    full = oracle.prefill(q, k, v, 0, base, k_turns)
    for h in range(6):
        one = oracle.prefill(q[:, h:h + 1], k[:, h // 3:h // 3 + 1], v[:, h // 3:h // 3 + 1], 0, base, k_turns)
        np.testing.assert_array_equal(one[:, 0], full[:, h])
    # an explicit head map is honoured
    hmap = [1, 0, 1, 0, 1, 0]
    mapped = oracle.prefill(q, k, v, 0, base, k_turns, kv_head_of_q=hmap)
    for h in range(6):
        one = oracle.prefill(q[:, h:h + 1], k[:, hmap[h]:hmap[h] + 1], v[:, hmap[h]:hmap[h] + 1], 0, base,
                             k_turns)
        np.testing.assert_array_equal(one[:, 0], mapped[:, h])


def test_row_subsets_match_full():
    d, base, k_turns, n = 16, 1e4, 0.5, 40
    q, k, v = _rand((2, 2, n, d), 32), _rand((2, 1, n, d), 33), _rand((2, 1, n, d), 34)
    full = oracle.prefill(q, k, v, 0, base, k_turns)
    rows = [0, 5, 39]
    sub = oracle.prefill(q, k, v, 0, base, k_turns, query_rows=rows, heads=[1], batches=[1])
    np.testing.assert_array_equal(sub[0, 0], full[1, 1, rows])


# ---------------------------------------------------------------- planted mistakes
# Each mutant is a plausible slip in the oracle; at least one pin above must
# reject it.  The mutation is applied on the CPU to the oracle only.

def _rope_wrong_sign(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)


def _rope_interleaved(x, positions, theta):
    x = np.asarray(x, dtype=np.float64)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x2 * c + x1 * s
    return out


def test_planted_rotation_mistakes_are_caught(monkeypatch):
    for bad in (_rope_wrong_sign, _rope_interleaved):
        monkeypatch.setattr(attention, "rope", bad)
        with pytest.raises(AssertionError):
            test_window_off_equals_textbook(25, 15, 40, True)
        with pytest.raises(AssertionError):
            test_scalar_triple_loop(0, 9, 9, True)
        monkeypatch.undo()


def test_planted_boundary_mistake_is_caught(monkeypatch):
    real = window.window_widths

    def exclusive(head_dim, rope_base, k_turns, window_on=True, scaling=None):   # keeps delta < W, not <= W
        w = real(head_dim, rope_base, k_turns, window_on, scaling)
        return np.where(w == window.UNBOUNDED, w, w - 1)

    monkeypatch.setattr(attention, "window_widths", exclusive)
    with pytest.raises(AssertionError):
        test_scalar_triple_loop(0, 9, 9, True)


def test_planted_scale_mistake_is_caught(monkeypatch):
    real = attention._row_output

    def no_scale(q_hat, q_pos, k_hat, v, k_pos, widths, scale, causal, allowed=None):
        return real(q_hat, q_pos, k_hat, v, k_pos, widths, 1.0, causal, allowed)

    monkeypatch.setattr(attention, "_row_output", no_scale)
    with pytest.raises(AssertionError):
        test_window_off_equals_torch_sdpa()
