"""Pins of the oracle's block-sparse composition: a token-level (block)
selection decides which keys a query attends, and the per-pair window applies
on top of it inside that set ("ATFlash: Per-RoPE-Wavelength Attention Windows
for Compute/Memory-Efficient LLM Inference", arXiv abstract: token-level
selection is orthogonal to the frequency-level pruning).

Pinned against: a pure-Python scalar loop over (query, key, pair) with the
selection test written out; torch's scaled_dot_product_attention with a
boolean mask (window off, complex-number RoPE route); the dense oracle (all
blocks selected); brute-force enumeration of the attended cells for the
counts."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import window


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _selection(n_qb, n_kb, density, seed, diagonal=True):
    sel = np.random.default_rng(seed).random((n_qb, n_kb)) < density
    if diagonal:
        for i in range(min(n_qb, n_kb)):
            sel[i, i] = True
    return sel


def _scalar_loops_selected(q, k, v, q_pos0, base, k_turns, causal, sel, block):
    """Pure-Python loop: query i attends key m iff sel[i // block][m // block]
    (and m <= position when causal); inside, pair r counts iff |n - m| <= W_r."""
    n_q, d = len(q), len(q[0])
    h = d // 2
    scale = 1 / math.sqrt(d)
    out = []
    for i in range(n_q):
        n = q_pos0 + i
        scores, vals = [], []
        for m in range(len(k)):
            if not sel[i // block][m // block]:
                continue
            if causal and m > n:
                continue
            s = 0.0
            for r in range(h):
                th = base ** (-2.0 * r / d)
                if abs(n - m) > math.floor(k_turns * 2 * math.pi / th):
                    continue
                a, b = n * th, m * th
                q1 = q[i][r] * math.cos(a) - q[i][r + h] * math.sin(a)
                q2 = q[i][r + h] * math.cos(a) + q[i][r] * math.sin(a)
                k1 = k[m][r] * math.cos(b) - k[m][r + h] * math.sin(b)
                k2 = k[m][r + h] * math.cos(b) + k[m][r] * math.sin(b)
                s += q1 * k1 + q2 * k2
            scores.append(scale * s)
            vals.append(v[m])
        if not scores:
            out.append([0.0] * d)
            continue
        mx = max(scores)
        ps = [math.exp(s - mx) for s in scores]
        tot = sum(ps)
        out.append([sum(p * vv[c] for p, vv in zip(ps, vals)) / tot for c in range(d)])
    return np.array(out)


@pytest.mark.parametrize("q_pos0,n_q,n_kv,causal", [(0, 12, 12, True), (3, 9, 14, True), (0, 8, 11, False)])
def test_scalar_loop_with_selection(q_pos0, n_q, n_kv, causal):
    d, base, k_turns, block = 6, 10.0, 0.3, 3       # windows [1, 4, 8]: pruning is active
    assert list(window.window_widths(d, base, k_turns)) == [1, 4, 8]
    sel = _selection(-(-n_q // block), -(-n_kv // block), 0.5, 40 + n_q)
    sel[1, :] = False                                 # a query block that attends nothing
    q, k, v = _rand((n_q, d), 41), _rand((n_kv, d), 42), _rand((n_kv, d), 43)
    out = oracle.prefill(q[None, None], k[None, None], v[None, None], q_pos0, base, k_turns,
                         causal=causal, key_blocks=sel[None, None], block=block)[0, 0]
    ref = _scalar_loops_selected(q.tolist(), k.tolist(), v.tolist(), q_pos0, base, k_turns, causal,
                                 sel.tolist(), block)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    assert np.all(out[block:2 * block] == 0.0)


def _cplx(x):
    h = x.shape[-1] // 2
    return x[..., :h] + 1j * x[..., h:]


def _rope_complex(x, pos, theta):
    z = _cplx(np.asarray(x, dtype=np.float64))
    zr = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :])
    return np.concatenate([zr.real, zr.imag], axis=-1)


def test_window_off_equals_sdpa_with_block_mask():
    d, base, n, block = 32, 1e4, 100, 16
    nb = -(-n // block)
    sel = _selection(nb, nb, 0.3, 44)                  # diagonal kept: every row attends a key
    q, k, v = _rand((1, 1, n, d), 45), _rand((1, 1, n, d), 46), _rand((1, 1, n, d), 47)
    out = oracle.prefill(q, k, v, 0, base, 4.0, window_on=False, key_blocks=sel[None, None],
                         block=block)
    theta = window.pair_frequencies(d, base)
    qh = torch.tensor(_rope_complex(q[0, 0], np.arange(n), theta))[None, None]
    kh = torch.tensor(_rope_complex(k[0, 0], np.arange(n), theta))[None, None]
    idx = np.arange(n)
    mask = (idx[None, :] <= idx[:, None]) & sel[idx[:, None] // block, idx[None, :] // block]
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh, torch.tensor(v), attn_mask=torch.tensor(mask))
    np.testing.assert_allclose(out, ref.numpy(), atol=1e-12)


def test_all_blocks_selected_is_dense_bitwise():
    d, base, n = 64, 1e4, 150
    q, k, v = _rand((1, 2, n, d), 48), _rand((1, 1, n, d), 49), _rand((1, 1, n, d), 50)
    nb = -(-n // 64)
    sel = np.ones((1, 2, nb, nb), dtype=bool)
    a = oracle.prefill(q, k, v, 0, base, 2.0, key_blocks=sel)
    b = oracle.prefill(q, k, v, 0, base, 2.0)
    assert np.array_equal(a, b)


COUNT_CASES = [(13, 13, 0, True, 4), (9, 17, 8, True, 3), (11, 14, 0, False, 4), (70, 130, 60, True, 16),
               (64, 200, 0, False, 32), (100, 100, 0, True, 64)]


@pytest.mark.parametrize("n_q,n_kv,q_pos0,causal,block", COUNT_CASES)
@pytest.mark.parametrize("d,base,k_turns", [(8, 10.0, 0.3), (64, 1e4, 1.0)])
def test_block_counts_match_bruteforce(n_q, n_kv, q_pos0, causal, block, d, base, k_turns):
    sel = _selection(-(-n_q // block), -(-n_kv // block), 0.45, n_q * 7 + n_kv, diagonal=False)
    a = oracle.pruned_terms_blocks(n_q, n_kv, q_pos0, d, base, k_turns, sel, causal, block=block)
    b = oracle.pruned_terms_blocks_bruteforce(n_q, n_kv, q_pos0, d, base, k_turns, sel, causal,
                                              block=block)
    assert a == b
    assert 0 <= a[0] <= a[1]


@pytest.mark.parametrize("n_q,n_kv,q_pos0,causal,block", COUNT_CASES)
def test_block_counts_all_selected_equal_dense(n_q, n_kv, q_pos0, causal, block):
    sel = np.ones((-(-n_q // block), -(-n_kv // block)), dtype=bool)
    a = oracle.pruned_terms_blocks(n_q, n_kv, q_pos0, 16, 50.0, 1.0, sel, causal, block=block)
    assert a == oracle.pruned_terms(n_q, n_kv, q_pos0, 16, 50.0, 1.0, causal)
    none = np.zeros_like(sel)
    assert oracle.pruned_terms_blocks(n_q, n_kv, q_pos0, 16, 50.0, 1.0, none, causal, block=block) == (0, 0)


@pytest.mark.parametrize("causal", [True, False])
def test_decode_with_selection_equals_prefill_row(causal):
    """The decode oracle with a per-(sequence, kv head) selection gives the
    prefill oracle's row for the same query, keys and selection."""
    d, base, k_turns, block = 32, 1e4, 1.0, 16
    kv_len, h_q, h_kv = [150, 97], 4, 2
    q = _rand((2, h_q, d), 51)
    kc, vc = _rand((2, h_kv, 160, d), 52), _rand((2, h_kv, 160, d), 53)
    sel = np.random.default_rng(54).random((2, h_kv, 10)) < 0.5
    sel[1, 1] = False                                  # a head that attends nothing
    q_pos = [149, 130]
    out = oracle.decode(q, kc, vc, kv_len, q_pos, base, k_turns, causal=causal, key_blocks=sel, block=block)
    for b in range(2):
        for hq in range(h_q):
            kvh = hq // (h_q // h_kv)
            n = kv_len[b]
            kb = sel[b, kvh][None, None, None, :-(-n // block)]
            ref = oracle.prefill(q[b, hq][None, None, None], kc[b, kvh][None, None, :n], vc[b, kvh][None, None, :n],
                                 q_pos[b], base, k_turns, causal=causal, key_blocks=kb, block=block)[0, 0, 0]
            np.testing.assert_array_equal(out[b, hq], ref)
    assert np.all(out[1, 2:] == 0.0)
