"""GPU parity of atw_prefill against the fp64 oracle (through the C ABI).

Floating point: max abs error <= 1e-4 (fp32 inputs) / <= 1e-2 (bf16 inputs).
Integers (device tile plans, per-tile pruned counts): bit-exact.
Gates: window on with nothing pruned == window off, bit for bit; two runs are
bit-identical.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import (BF16_TOL, bf16_err, F32_TOL, ROW_ABS, ROW_REL, check_rows, max_err, sample_rows, say,
                            sync, to_np)

pytestmark = pytest.mark.gpu


def _run_and_compare(q, k, v, base, k_turns, tol, q_pos0=0, causal=True, window_on=True,
                     kv_head_of_q=None, rows=None):
    out = atw.prefill(q, k, v, rope_base=base, k_turns=k_turns, q_pos0=q_pos0, causal=causal,
                      window_on=window_on, kv_head_of_q=kv_head_of_q)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), q_pos0, base, k_turns, causal=causal,
                         window_on=window_on, kv_head_of_q=kv_head_of_q, query_rows=rows)
    got = to_np(out) if rows is None else to_np(out)[:, :, rows]
    err = bf16_err(got, ref) if tol == BF16_TOL else max_err(got, ref)
    say(f"  max abs err {err:.3e} (tol {tol})")
    assert np.isfinite(got).all()
    assert err <= tol
    return out, ref


@pytest.mark.parametrize("window_on", [True, False])
def test_single_head_fp32_1k(window_on):
    """The fp32 single-head workload: N=1024, d=64, base 1e4, k=4, full output."""
    w = synth.WORKLOADS["single-head-1k"]
    say(f"prefill fp32 1k window_on={window_on}")
    q, k, v = synth.prefill_inputs(1, 1, 1, 1024, 1024, 64, torch.float32, w.seed, device="cuda",
                                   gen_device="cpu")
    _run_and_compare(q, k, v, w.rope_base, w.k_turns, F32_TOL, window_on=window_on)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("k_turns", [0.35, 4.0])
def test_bf16_ragged_gqa(d, k_turns):
    """Several 256-row blocks and 64-key tiles with ragged tails, GQA 2:1,
    windows short enough that most tiles have partially windowed pairs."""
    say(f"prefill bf16 ragged d={d} k={k_turns}")
    q, k, v = synth.prefill_inputs(2, 4, 2, 700, 700, d, torch.bfloat16, 7, device="cuda")
    _run_and_compare(q, k, v, 1e4, k_turns, BF16_TOL)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("k_turns", [0.35, 4.0])
def test_bf16_seed_sweep(d, k_turns):
    """The ragged 700-row GQA case over 32 seeds (stops at the first failure):
    the 1e-2 bar holds on every draw, not on a chosen one."""
    for seed in range(1000, 1032):
        q, k, v = synth.prefill_inputs(1, 4, 2, 700, 700, d, torch.bfloat16, seed, device="cuda")
        out = atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns)
        sync()
        ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, k_turns)
        got = to_np(out)
        err = bf16_err(got, ref)
        say(f"  seed {seed} d={d} k={k_turns}: max abs err {err:.3e}")
        assert np.isfinite(got).all() and err <= BF16_TOL, (seed, err)


@pytest.mark.parametrize("d", [64, 128])
def test_every_pair_pruned_in_far_tiles(d):
    """Windows so short (k = 0.02) that beyond ~1000 positions every pair is
    pruned: far cells score 0 and stay in the softmax; whole workgroups then
    copy no K' block of a tile and read zeroed / stale K' slots against a fully
    masked query operand."""
    say(f"prefill bf16 every pair pruned far away, d={d}")
    assert oracle.window_widths(d, 1e4, 0.02)[-1] < 1200
    q, k, v = synth.prefill_inputs(1, 2, 1, 3000, 3000, d, torch.bfloat16, 16, device="cuda")
    _run_and_compare(q, k, v, 1e4, 0.02, BF16_TOL)
    # and the fp32 path
    q, k, v = synth.prefill_inputs(1, 2, 1, 2100, 2100, d, torch.float32, 17, device="cuda")
    _run_and_compare(q, k, v, 1e4, 0.02, F32_TOL)


def test_fp32_ragged_d128_partial_pairs():
    say("prefill fp32 ragged d=128")
    q, k, v = synth.prefill_inputs(1, 2, 1, 333, 333, 128, torch.float32, 8, device="cuda")
    _run_and_compare(q, k, v, 100.0, 0.3, F32_TOL)


def test_chunked_prefill_q_pos0():
    """A query chunk at positions 500.. against the whole prefix (chunked prefill)."""
    say("prefill bf16 chunk q_pos0=500")
    q, k, v = synth.prefill_inputs(1, 2, 2, 300, 800, 64, torch.bfloat16, 9, device="cuda")
    _run_and_compare(q, k, v, 1e4, 0.5, BF16_TOL, q_pos0=500)


def test_chunked_equals_one_shot_on_gpu():
    say("prefill bf16 chunked == one-shot")
    q, k, v = synth.prefill_inputs(1, 2, 1, 640, 640, 128, torch.bfloat16, 10, device="cuda")
    full = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.5)
    parts = []
    for s in range(0, 640, 256):
        e = min(640, s + 256)
        parts.append(atw.prefill(q[:, :, s:e], k[:, :, :e], v[:, :, :e], rope_base=1e4, k_turns=0.5,
                                 q_pos0=s))
    sync()
    # same rows, same keys, same tiles -> same arithmetic
    assert torch.equal(torch.cat(parts, dim=2), full)


def test_non_causal():
    say("prefill bf16 non-causal")
    q, k, v = synth.prefill_inputs(1, 2, 1, 200, 333, 64, torch.bfloat16, 11, device="cuda")
    _run_and_compare(q, k, v, 1e4, 0.5, BF16_TOL, causal=False)


def test_explicit_head_map_and_strides():
    """kv_head_of_q given explicitly, inputs in token-major [B, N, H, d] storage."""
    say("prefill bf16 head map + token-major strides")
    g = synth.generator(12)
    qs = torch.randn((1, 300, 6, 128), generator=g).to(torch.bfloat16).cuda()
    ks = torch.randn((1, 300, 3, 128), generator=g).to(torch.bfloat16).cuda()
    vs = torch.randn((1, 300, 3, 128), generator=g).to(torch.bfloat16).cuda()
    q, k, v = qs.transpose(1, 2), ks.transpose(1, 2), vs.transpose(1, 2)
    hmap = [2, 0, 1, 1, 0, 2]
    _run_and_compare(q, k, v, 1e4, 1.0, BF16_TOL, kv_head_of_q=hmap)


def test_nothing_pruned_is_window_off_bitwise():
    """Gate: with W_0 >= N-1 the window removes nothing, and the result must be
    bit-identical to window off (the analogue of the pages' bit-identity gate)."""
    say("gate: nothing pruned == off")
    q, k, v = synth.prefill_inputs(1, 2, 2, 600, 600, 128, torch.bfloat16, 13, device="cuda")
    k_turns = 100.0
    assert oracle.window_widths(128, 1e4, k_turns)[0] >= 599
    on = atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns, window_on=True)
    off = atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns, window_on=False)
    inf = atw.prefill(q, k, v, rope_base=1e4, k_turns=math.inf, window_on=True)
    sync()
    assert torch.equal(on, off)
    assert torch.equal(inf, off)


def test_deterministic():
    say("gate: determinism")
    q, k, v = synth.prefill_inputs(1, 4, 2, 513, 513, 128, torch.bfloat16, 14, device="cuda")
    a = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.7)
    b = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.7)
    sync()
    assert torch.equal(a, b)


def test_empty_and_tiny():
    say("prefill edge: n_q=0, n=1, n=2")
    q, k, v = synth.prefill_inputs(1, 1, 1, 0, 5, 64, torch.bfloat16, 15, device="cuda")
    out = atw.prefill(q, k, v, rope_base=1e4, k_turns=4.0)
    assert out.numel() == 0
    for n in (1, 2, 65):
        q, k, v = synth.prefill_inputs(1, 1, 1, n, n, 64, torch.bfloat16, 16 + n, device="cuda")
        _run_and_compare(q, k, v, 1e4, 0.2, BF16_TOL)


@pytest.mark.parametrize("case", [
    dict(n_q=700, n_kv=700, p0=0, causal=True, tq=32, tk=64, d=128, base=1e4, k=0.35),
    dict(n_q=256, n_kv=1300, p0=1044, causal=True, tq=32, tk=64, d=64, base=1e6, k=8.0),
    dict(n_q=200, n_kv=333, p0=0, causal=False, tq=32, tk=64, d=64, base=1e4, k=0.5),
    dict(n_q=1000, n_kv=1000, p0=0, causal=True, tq=17, tk=23, d=32, base=100.0, k=0.4),
    # the workgroup x key-tile geometry the bf16 prefill stages by (head_dim
    # 128: 12 waves x 32 rows; head_dim 64: 8 waves x 32 rows)
    dict(n_q=1000, n_kv=1000, p0=0, causal=True, tq=384, tk=64, d=128, base=1e4, k=0.35),
    dict(n_q=700, n_kv=1500, p0=800, causal=True, tq=256, tk=64, d=64, base=1e4, k=0.5),
])
def test_device_plan_bit_exact(case):
    """Per-tile pair ranges and pruned counts from the kernels' device code equal
    the oracle's brute force exactly, and the counts sum to the closed form."""
    say(f"device plan {case}")
    c = case
    plan, pruned = atw.window_plan_device(c["d"], c["base"], c["k"], True, c["n_q"], c["n_kv"], c["p0"],
                                          c["causal"], c["tq"], c["tk"])
    sync()
    w = oracle.window_widths(c["d"], c["base"], c["k"])
    ref = oracle.tile_plan(c["n_q"], c["n_kv"], c["p0"], c["causal"], c["tq"], c["tk"], w)
    np.testing.assert_array_equal(plan.cpu().numpy(), ref)
    total_pruned = int(pruned.sum().item())
    exp = oracle.pruned_terms_bruteforce(c["n_q"], c["n_kv"], c["p0"], c["d"], c["base"], c["k"],
                                         c["causal"], True)[0]
    assert total_pruned == exp


def test_device_plan_workload_count():
    """Device count at the 32K Qwen2.5-0.5B shape equals the exact closed form."""
    say("device plan 32k")
    plan, pruned = atw.window_plan_device(64, 1e6, 8.0, True, 32768, 32768, 0, True, 32, 64)
    sync()
    assert int(pruned.sum().item()) == oracle.pruned_terms(32768, 32768, 0, 64, 1e6, 8.0)[0]


def _workload_rows_check(name, n_rows_random=6, heads=None):
    w = synth.WORKLOADS[name]
    say(f"workload {name}: generating inputs")
    q, k, v = synth.workload_prefill_inputs(w)
    say(f"workload {name}: running window on/off")
    on = atw.prefill(q, k, v, rope_base=w.rope_base, k_turns=w.k_turns, window_on=True)
    off = atw.prefill(q, k, v, rope_base=w.rope_base, k_turns=w.k_turns, window_on=False)
    sync()
    wid = oracle.window_widths(w.head_dim, w.rope_base, w.k_turns)
    rows = sample_rows(w.n, extra=[int(x) + 1 for x in wid[:6]], seed=w.seed, count=n_rows_random)
    heads = heads or [0, w.h_q // w.h_kv - 1, w.h_q // w.h_kv, w.h_q - 1]
    G = w.h_q // w.h_kv
    kvs = sorted({h // G for h in heads})
    qn = to_np(q[:, heads][:, :, rows])
    kn, vn = to_np(k[:, kvs]), to_np(v[:, kvs])
    hmap = [kvs.index(h // G) for h in heads]
    say(f"workload {name}: oracle on {len(rows)} rows x {len(heads)} heads")
    for window_on, out in ((True, on), (False, off)):
        ref = np.zeros((1, len(heads), len(rows), w.head_dim))
        for i, r in enumerate(rows):
            ref[:, :, i] = oracle.prefill(qn[:, :, i:i + 1], kn[:, :, :r + 1], vn[:, :, :r + 1], r,
                                          w.rope_base, w.k_turns, window_on=window_on,
                                          kv_head_of_q=hmap)[:, :, 0]
        got = to_np(out[:, heads][:, :, rows])
        check_rows(got, ref, f"window_on={window_on}")
        if window_on:
            ref_on, got_on = ref, got
        else:
            # the window's effect itself matches: (on - off) against the
            # oracle's difference, per row relative to the row's outputs
            diff_err = max_err(got_on - got, ref_on - ref)
            row_err = np.abs((got_on - got) - (ref_on - ref)).max(axis=-1)
            bound = 2 * (ROW_REL * np.maximum(np.abs(ref_on).max(axis=-1), np.abs(ref).max(axis=-1)) + ROW_ABS)
            say(f"  (on - off) max abs err {diff_err:.3e}, worst row ratio {float((row_err / bound).max()):.3f}")
            assert diff_err <= 2 * BF16_TOL
            assert (row_err <= bound).all()


def test_workload_qwen_32k_sampled_rows():
    _workload_rows_check("qwen2.5-0.5b-32k")


def test_workload_llama_128k_sampled_rows():
    _workload_rows_check("llama-3.2-3b-128k", n_rows_random=3, heads=[0, 23])


@pytest.mark.parametrize("n_q,q_pos0", [(127, 0), (255, 0), (256, 0), (257, 0), (383, 0), (384, 0), (385, 0),
                                        (769, 200)])
def test_workgroup_row_boundaries(n_q, q_pos0):
    """Query counts at and around one workgroup (head_dim 128: 12 waves of 32
    rows = 384 rows; head_dim 64: 8 waves = 256 rows), a last wave with 31
    rows (127), and a chunk offset in the last case: the last workgroup's
    idle waves and rows must not disturb the rest."""
    say(f"prefill bf16 d=128 n_q={n_q} q_pos0={q_pos0}")
    n_kv = n_q + q_pos0
    q, k, v = synth.prefill_inputs(1, 3, 1, n_q, n_kv, 128, torch.bfloat16, 90 + n_q, device="cuda")
    _run_and_compare(q, k, v, 1e4, 0.5, BF16_TOL, q_pos0=q_pos0)
    q64, k64, v64 = synth.prefill_inputs(1, 2, 1, n_q, n_kv, 64, torch.bfloat16, 91 + n_q, device="cuda")
    _run_and_compare(q64, k64, v64, 1e4, 0.5, BF16_TOL, q_pos0=q_pos0)
