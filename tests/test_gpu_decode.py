"""GPU parity of atw_decode (split-KV + combine) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import BF16_TOL, bf16_err, check_rows, max_err, say, sync, to_np

pytestmark = pytest.mark.gpu


def _check(q, kc, vc, kv_len, q_pos, base, k_turns, splits, causal=True, window_on=True, heads=None,
           batches=None, kv_head_of_q=None):
    out = atw.decode(q, kc, vc, kv_len, q_pos, rope_base=base, k_turns=k_turns, causal=causal,
                     window_on=window_on, num_splits=splits, kv_head_of_q=kv_head_of_q)
    sync()
    batches = batches or list(range(q.shape[0]))
    heads = heads or list(range(q.shape[1]))
    ref = oracle.decode(to_np(q[batches]), to_np(kc[batches]), to_np(vc[batches]),
                        [kv_len[b] for b in batches], [q_pos[b] for b in batches], base, k_turns,
                        causal=causal, window_on=window_on, heads=heads, kv_head_of_q=kv_head_of_q)
    got = to_np(out[batches][:, heads])
    err = bf16_err(got, ref)
    say(f"  splits={splits} max abs err {err:.3e}")
    assert np.isfinite(got).all()
    assert err <= BF16_TOL
    return out


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 7, 64])
def test_decode_ragged_batch(d, splits):
    say(f"decode ragged d={d} splits={splits}")
    q, kc, vc = synth.decode_inputs(3, 8, 2, 1100, d, torch.bfloat16, 21, device="cuda")
    kv_len = [1100, 777, 33]
    q_pos = [1099, 776 + 50, 32]      # sequence 1: query ahead of its cache (all keys visible)
    _check(q, kc, vc, kv_len, q_pos, 1e4, 0.5, splits)


def test_decode_window_off_and_nothing_pruned():
    say("decode window off / nothing pruned")
    q, kc, vc = synth.decode_inputs(2, 4, 1, 600, 128, torch.bfloat16, 22, device="cuda")
    off = _check(q, kc, vc, [600, 600], [600, 600], 1e4, 4.0, 8, window_on=False)
    on = atw.decode(q, kc, vc, [600, 600], [600, 600], rope_base=1e4, k_turns=100.0, num_splits=8)
    sync()
    assert torch.equal(on, off)


def test_decode_non_causal_and_head_map():
    say("decode non-causal + head map")
    q, kc, vc = synth.decode_inputs(1, 6, 3, 500, 128, torch.bfloat16, 23, device="cuda")
    _check(q, kc, vc, [500], [200], 1e4, 0.5, 5, causal=False, kv_head_of_q=[2, 2, 0, 1, 0, 1])


def test_decode_fewer_query_heads_than_kv_heads():
    """An explicit head map may leave kv heads unread (2 query heads over 4
    kv heads): those kv heads' waves have no columns, and the query heads
    still read their own kv heads -- also with the heads in model order of a
    default-looking prefix (query head 0 -> kv head 0)."""
    say("decode h_q < h_kv with a head map")
    q, kc, vc = synth.decode_inputs(2, 2, 4, 300, 128, torch.bfloat16, 24, device="cuda")
    for hmap in ([3, 1], [0, 2], [0, 1]):
        _check(q, kc, vc, [300, 211], [299, 210], 1e4, 0.5, 3, kv_head_of_q=hmap)
    q, kc, vc = synth.decode_inputs(1, 6, 3, 300, 64, torch.bfloat16, 25, device="cuda")
    _check(q, kc, vc, [300], [299], 1e4, 0.5, 4, kv_head_of_q=[0, 0, 1, 1, 2, 2])   # in order, given


def test_decode_row_equals_prefill_row():
    """A decode step at position n against keys 0..n equals prefill row n."""
    say("decode row == prefill row")
    q, k, v = synth.prefill_inputs(1, 4, 2, 400, 400, 128, torch.bfloat16, 24, device="cuda")
    pre = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.5)
    for n in (0, 63, 255, 399):
        dec = atw.decode(q[:, :, n], k, v, [n + 1], [n], rope_base=1e4, k_turns=0.5, num_splits=3)
        sync()
        assert max_err(to_np(dec), to_np(pre[:, :, n]).astype(np.float64)) <= 2 * BF16_TOL


def test_decode_workload_512k_sampled():
    """Qwen2.5-7B-1M-shaped decode: B=8, 28/4 heads, L=524288, 64 splits.
    The oracle checks every query head of three (sequence, kv head) pairs."""
    w = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
    say("decode 512k: generating inputs")
    q, kc, vc = synth.workload_decode_inputs(w)
    L = w.n
    say("decode 512k: running")
    out_on = atw.decode(q, kc, vc, [L] * 8, [L] * 8, rope_base=w.rope_base, k_turns=w.k_turns,
                        num_splits=w.splits)
    out_off = atw.decode(q, kc, vc, [L] * 8, [L] * 8, rope_base=w.rope_base, k_turns=w.k_turns,
                         num_splits=w.splits, window_on=False)
    sync()
    G = w.h_q // w.h_kv
    for b, kvh in ((0, 0), (3, 2), (7, 3)):
        heads = list(range(kvh * G, (kvh + 1) * G))
        qn = to_np(q[b:b + 1, heads])
        kn, vn = to_np(kc[b:b + 1, kvh:kvh + 1]), to_np(vc[b:b + 1, kvh:kvh + 1])
        say(f"decode 512k: oracle b={b} kv={kvh}")
        for window_on, out in ((True, out_on), (False, out_off)):
            ref = oracle.decode(qn, kn, vn, [L], [L], w.rope_base, w.k_turns, window_on=window_on,
                                kv_head_of_q=[0] * G)
            check_rows(to_np(out[b:b + 1, heads]), ref, f"window_on={window_on}")


def _band_ref(kc):
    """Pair-banded copy of a row cache by tensor indexing: band c of key m is
    dims [8c, 8c+8) then [h+8c, h+8c+8)."""
    B, H, L, D = kc.shape
    h = D // 2
    lo = kc[..., :h].reshape(B, H, L, D // 16, 8)
    hi = kc[..., h:].reshape(B, H, L, D // 16, 8)
    return torch.cat([lo, hi], dim=-1).permute(0, 1, 3, 2, 4).contiguous()


@pytest.mark.parametrize("d", [64, 128])
def test_kcache_band_exact(d):
    say(f"kcache band d={d}")
    _, kc, _ = synth.decode_inputs(2, 4, 3, 1000, d, torch.bfloat16, 25, device="cuda")
    bands = atw.kcache_band(kc)
    sync()
    assert torch.equal(bands, _band_ref(kc))
    # append in two steps into a strided (padded) buffer: [0, 700) then [700, 1000)
    buf = torch.zeros((2, 3, d // 16, 1024, 16), dtype=torch.bfloat16, device="cuda")
    atw.kcache_band(kc, buf, t0=0, n_tokens=700)
    atw.kcache_band(kc, buf, t0=700, n_tokens=300)
    sync()
    assert torch.equal(buf[:, :, :, :1000], _band_ref(kc))
    assert not buf[:, :, :, 1000:].any()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("splits", [1, 7, 64])
def test_decode_banded_ragged_batch(d, splits):
    """Banded cache: parity with the oracle (its splits are sized by bytes, so
    they differ from the row layout's); bit-identity with the row layout when
    the window is off (equal splits on both)."""
    say(f"decode banded ragged d={d} splits={splits}")
    q, kc, vc = synth.decode_inputs(3, 8, 2, 1100, d, torch.bfloat16, 21, device="cuda")
    kv_len = [1100, 777, 33]
    q_pos = [1099, 776 + 50, 32]
    bands = atw.kcache_band(kc)
    got = atw.decode_banded(q, bands, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.5,
                            num_splits=splits)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.5)
    err = bf16_err(to_np(got), ref)
    say(f"  banded max abs err {err:.3e}")
    assert err <= BF16_TOL
    rows = atw.decode(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.5, window_on=False,
                      num_splits=splits)
    got = atw.decode_banded(q, bands, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.5,
                            window_on=False, num_splits=splits)
    sync()
    assert torch.equal(got, rows)


def test_decode_banded_non_causal_window_off_head_map():
    say("decode banded non-causal / window off / head map")
    q, kc, vc = synth.decode_inputs(1, 6, 3, 500, 128, torch.bfloat16, 23, device="cuda")
    bands = atw.kcache_band(kc)
    hm = [2, 2, 0, 1, 0, 1]
    for causal, window_on, qp in ((False, True, 200), (True, True, 499), (True, False, 499)):
        got = atw.decode_banded(q, bands, vc, [500], [qp], rope_base=1e4, k_turns=0.5,
                                causal=causal, window_on=window_on, num_splits=5, kv_head_of_q=hm)
        sync()
        ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), [500], [qp], 1e4, 0.5, causal=causal,
                            window_on=window_on, kv_head_of_q=hm)
        err = bf16_err(to_np(got), ref)
        say(f"  causal={causal} window_on={window_on} max abs err {err:.3e}")
        assert err <= BF16_TOL


def test_decode_banded_workload_512k_sampled():
    """The 512K decode workload over a banded cache: one (sequence, kv head)
    against the oracle, every output against the row-layout result."""
    w = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
    say("decode banded 512k: generating inputs")
    q, kc, vc = synth.workload_decode_inputs(w)
    L = w.n
    G = w.h_q // w.h_kv
    b, kvh = 5, 1
    heads = list(range(kvh * G, (kvh + 1) * G))
    k_rows = to_np(kc[b:b + 1, kvh:kvh + 1])
    say("decode banded 512k: running")
    rows = atw.decode(q, kc, vc, [L] * 8, [L] * 8, rope_base=w.rope_base, k_turns=w.k_turns,
                      num_splits=w.splits)
    bands = atw.kcache_band(kc)
    del kc
    got = atw.decode_banded(q, bands, vc, [L] * 8, [L] * 8, rope_base=w.rope_base,
                            k_turns=w.k_turns, num_splits=w.splits)
    sync()
    assert max_err(to_np(got), to_np(rows).astype(np.float64)) <= 2 * BF16_TOL
    say(f"decode banded 512k: oracle b={b} kv={kvh}")
    ref = oracle.decode(to_np(q[b:b + 1, heads]), k_rows, to_np(vc[b:b + 1, kvh:kvh + 1]), [L], [L],
                        w.rope_base, w.k_turns, kv_head_of_q=[0] * G)
    check_rows(to_np(got[b:b + 1, heads]), ref, "banded")
