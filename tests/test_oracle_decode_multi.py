"""Pins for oracle.decode_multi (several query tokens per sequence).

Draft tokens of multi-token prediction sit at consecutive positions and each
attends causally with the window measured from its own position
("ATFlash — Per-RoPE-Wavelength Attention Windows", README, "MiMo-V2.6-Pro-RL
and MTP" for the drafts under the window; "The idea": the window of a pair
depends on the query-key distance only).  Pinned here against:

* a pure-Python scalar loop over (token, key, pair) with the rotation written
  out per element (no oracle code);
* the single-token decode at position q_pos + j over keys 0 .. q_pos + j;
* the prefill rows at q_pos0 = q_pos (token j is prefill row j);
* planted mistakes (token j placed at q_pos, every token's window measured
  from token 0) that these pins must reject.

The windows are chosen short ([1, 4, 8] at d = 6) so that for some keys a
pair is kept at token 0's distance and dropped at a later token's.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import attention, window

D, BASE, K_TURNS = 6, 10.0, 0.3           # windows [1, 4, 8]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _scalar_multi(q, k, v, q_pos, n_kv, base, k_turns):
    """Token j of one head: scalar loop of the windowed definition at
    position q_pos + j over keys 0 .. min(n_kv, q_pos + j + 1) - 1."""
    n_tok, d = len(q), len(q[0])
    h = d // 2
    scale = 1 / math.sqrt(d)
    out = []
    for j in range(n_tok):
        n = q_pos + j
        scores, vals = [], []
        for m in range(min(n_kv, n + 1)):
            s = 0.0
            for r in range(h):
                th = base ** (-2.0 * r / d)
                if n - m > math.floor(k_turns * 2 * math.pi / th):
                    continue
                a, b = n * th, m * th
                q1 = q[j][r] * math.cos(a) - q[j][r + h] * math.sin(a)
                q2 = q[j][r + h] * math.cos(a) + q[j][r] * math.sin(a)
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


def _inputs(bsz=2, n_tok=4, h_q=4, h_kv=2, lmax=24, seed=40):
    q = _rand((bsz, n_tok, h_q, D), seed)
    k = _rand((bsz, h_kv, lmax, D), seed + 1)
    v = _rand((bsz, h_kv, lmax, D), seed + 2)
    return q, k, v


def test_windows_end_between_token_distances():
    # the case the pins below exercise: pair 0 (W = 1) kept at distance 1 and
    # dropped at distance 2, i.e. between tokens 0 and 1 for the key q_pos - 1
    assert list(window.window_widths(D, BASE, K_TURNS)) == [1, 4, 8]


@pytest.mark.parametrize("q_pos,kv_len", [([10, 5], [14, 9]), ([0, 3], [4, 7]), ([12, 12], [13, 24])])
def test_decode_multi_equals_scalar_loop(q_pos, kv_len):
    q, k, v = _inputs()
    out = attention.decode_multi(q, k, v, kv_len, q_pos, BASE, K_TURNS)
    for b in range(2):
        for hq in range(4):
            kvh = hq // 2
            ref = _scalar_multi(q[b, :, hq].tolist(), k[b, kvh].tolist(), v[b, kvh].tolist(),
                                q_pos[b], kv_len[b], BASE, K_TURNS)
            np.testing.assert_allclose(out[b, :, hq], ref, atol=1e-12)


def test_decode_multi_token_is_single_token_decode():
    q, k, v = _inputs(seed=50)
    q_pos, kv_len = [9, 15], [13, 20]
    out = attention.decode_multi(q, k, v, kv_len, q_pos, BASE, K_TURNS)
    for j in range(q.shape[1]):
        lens = [min(kv_len[b], q_pos[b] + j + 1) for b in range(2)]
        pos = [q_pos[b] + j for b in range(2)]
        ref = oracle.decode(q[:, j], k, v, lens, pos, BASE, K_TURNS)
        np.testing.assert_allclose(out[:, j], ref, atol=1e-12)


def test_decode_multi_tokens_are_prefill_rows():
    q, k, v = _inputs(seed=60)
    q_pos, kv_len = [7, 11], [11, 15]
    out = attention.decode_multi(q, k, v, kv_len, q_pos, BASE, K_TURNS)
    for b in range(2):
        # prefill rows at q_pos0 = q_pos[b]: row j at position q_pos[b] + j
        pre = oracle.prefill(np.transpose(q[b:b + 1], (0, 2, 1, 3)), k[b:b + 1, :, :kv_len[b]],
                             v[b:b + 1, :, :kv_len[b]], q_pos[b], BASE, K_TURNS)
        np.testing.assert_allclose(out[b], np.transpose(pre[0], (1, 0, 2)), atol=1e-12)


# ---------------------------------------------------------------- planted mistakes

def _multi_mutant(at_token0_position, window_from_token0):
    """decode_multi with one plausible slip: token j rotated and masked at
    q_pos (no + j), or every token's window measured from token 0."""

    def mutant(q, k_cache, v_cache, kv_len, q_pos, rope_base, k_turns, window_on=True, scale=None,
               kv_head_of_q=None, heads=None, batches=None, scaling=None):
        bsz, n_tok, h_q, d = q.shape
        h_kv = k_cache.shape[1]
        theta = window.pair_frequencies(d, rope_base)
        widths = window.window_widths(d, rope_base, k_turns, window_on)
        sc = 1.0 / math.sqrt(d)
        out = np.zeros((bsz, n_tok, h_q, d))
        for b in range(bsz):
            n_kv = int(kv_len[b])
            k_pos = np.arange(n_kv)
            for hq in range(h_q):
                kvh = hq // (h_q // h_kv)
                k_hat = attention.rope(k_cache[b, kvh, :n_kv], k_pos, theta)
                v64 = np.asarray(v_cache[b, kvh, :n_kv], dtype=np.float64)
                for j in range(n_tok):
                    pos = int(q_pos[b]) + (0 if at_token0_position else j)
                    q_hat = attention.rope(q[b, j, hq][None, :], np.array([pos]), theta)[0]
                    vis = k_pos <= pos
                    wpos = int(q_pos[b]) if window_from_token0 else pos
                    dist = wpos - k_pos[vis]
                    t = attention.pair_terms(q_hat, k_hat[vis])
                    s = sc * np.where(dist[:, None] <= widths[None, :], t, 0.0).sum(axis=1)
                    p = np.exp(s - s.max())
                    out[b, j, hq] = (p @ v64[vis]) / p.sum()
        return out

    return mutant


def test_mutant_harness_is_faithful(monkeypatch):
    # with neither slip the mutant is the definition itself: the pins pass
    monkeypatch.setattr(attention, "decode_multi", _multi_mutant(False, False))
    test_decode_multi_equals_scalar_loop([10, 5], [14, 9])
    test_decode_multi_token_is_single_token_decode()


@pytest.mark.parametrize("slip", [(True, False), (False, True)])
def test_planted_decode_multi_mistakes_are_caught(monkeypatch, slip):
    monkeypatch.setattr(attention, "decode_multi", _multi_mutant(*slip))
    with pytest.raises(AssertionError):
        test_decode_multi_equals_scalar_loop([10, 5], [14, 9])
    with pytest.raises(AssertionError):
        test_decode_multi_token_is_single_token_decode()
    with pytest.raises(AssertionError):
        test_decode_multi_tokens_are_prefill_rows()
