"""GPU parity with rescaled RoPE frequencies (model rope_scaling): prefill and
decode through the *_rope entry points against the fp64 oracle using the same
rule.  The rules are set so that all three bands of the llama3 rule (kept,
interpolated, blended) and short windows occur at these small sizes.  Explicit
window tables (zeros, windows inside and across key tiles, unbounded pairs)
go through prefill (bf16, fp32, block-sparse) and decode (rows and bands) with
k unused."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import BF16_TOL, bf16_err, F32_TOL, max_err, say, sync, to_np

pytestmark = pytest.mark.gpu

# plain wavelengths at base 1e4 span 6.3 .. 5.4e4 positions (d = 128), so with
# L = 256 the bands split at 64 and 256
SMALL_LLAMA3 = {"rope_type": "llama3", "factor": 4.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                "original_max_position_embeddings": 256}
LINEAR = {"rope_type": "linear", "factor": 3.0}


def _table(d, seed):
    rng = np.random.default_rng(seed)
    return {"rope_type": "table", "theta": list(np.sort(rng.uniform(1e-4, 1.5, d // 2))[::-1])}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("name", ["llama3", "linear", "table"])
def test_prefill_bf16_rope_scaling(d, name):
    sc = {"llama3": SMALL_LLAMA3, "linear": LINEAR, "table": _table(d, 3)}[name]
    say(f"prefill bf16 rope scaling {name} d={d}")
    q, k, v = synth.prefill_inputs(2, 4, 2, 700, 700, d, torch.bfloat16, 31, device="cuda")
    for k_turns in (0.4, 3.0):
        out = atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns, rope_scaling=sc)
        sync()
        ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, k_turns, scaling=sc)
        err = bf16_err(to_np(out), ref)
        say(f"  k={k_turns} max abs err {err:.3e}")
        assert np.isfinite(to_np(out)).all() and err <= BF16_TOL


def test_prefill_fp32_rope_scaling_chunk():
    say("prefill fp32 llama3 scaling, chunk at q_pos0 = 300")
    q, k, v = synth.prefill_inputs(1, 2, 1, 200, 500, 64, torch.float32, 32, device="cuda")
    out = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.7, q_pos0=300, rope_scaling=SMALL_LLAMA3)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 300, 1e4, 0.7, scaling=SMALL_LLAMA3)
    err = max_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert err <= F32_TOL


def test_scaling_changes_the_result():
    """The scaled path is not the plain one: outputs differ beyond tolerance."""
    q, k, v = synth.prefill_inputs(1, 2, 1, 400, 400, 128, torch.bfloat16, 33, device="cuda")
    a = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.5)
    b = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.5, rope_scaling=SMALL_LLAMA3)
    sync()
    assert max_err(to_np(a), to_np(b).astype(np.float64)) > 10 * BF16_TOL


@pytest.mark.parametrize("banded", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_rope_scaling(banded, d):
    say(f"decode rope scaling llama3 d={d} banded={banded}")
    q, kc, vc = synth.decode_inputs(2, 8, 2, 900, d, torch.bfloat16, 34, device="cuda")
    kv_len, q_pos = [900, 411], [899, 410]
    if banded:
        out = atw.decode_banded(q, atw.kcache_band(kc), vc, kv_len, q_pos, rope_base=1e4, k_turns=0.6,
                                num_splits=7, rope_scaling=SMALL_LLAMA3)
    else:
        out = atw.decode(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.6, num_splits=7,
                         rope_scaling=SMALL_LLAMA3)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.6, scaling=SMALL_LLAMA3)
    err = bf16_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert err <= BF16_TOL


def _explicit_widths(d, seed, top):
    """Non-decreasing windows that are not floor(k * lambda_r): zeros (only the
    diagonal keeps those pairs), windows inside one key tile, windows across
    tiles and unbounded pairs."""
    rng = np.random.default_rng(seed)
    h = d // 2
    w = np.sort(rng.integers(1, top, h))
    w[: h // 8] = 0
    w[h - h // 8:] = 1 << 62
    return [int(x) for x in w]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rule", [None, "llama3"])
def test_prefill_bf16_explicit_widths(d, rule):
    table = _explicit_widths(d, 40 + d, 600)
    sc = {"widths": table} if rule is None else dict(SMALL_LLAMA3, widths=table)
    say(f"prefill bf16 explicit widths d={d} rule={rule}")
    q, k, v = synth.prefill_inputs(2, 4, 2, 700, 700, d, torch.bfloat16, 41, device="cuda")
    out = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.0, rope_scaling=sc)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, 0.0, scaling=sc)
    err = bf16_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(to_np(out)).all() and err <= BF16_TOL


def test_prefill_fp32_explicit_widths_chunk():
    sc = {"widths": _explicit_widths(64, 42, 400)}
    say("prefill fp32 explicit widths, chunk at q_pos0 = 300")
    q, k, v = synth.prefill_inputs(1, 2, 1, 200, 500, 64, torch.float32, 43, device="cuda")
    out = atw.prefill(q, k, v, rope_base=1e4, k_turns=1.0, q_pos0=300, rope_scaling=sc)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 300, 1e4, 1.0, scaling=sc)
    err = max_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert err <= F32_TOL


@pytest.mark.parametrize("banded", [False, True])
def test_decode_explicit_widths(banded):
    d = 128
    sc = {"widths": _explicit_widths(d, 44, 800)}
    say(f"decode explicit widths d={d} banded={banded}")
    q, kc, vc = synth.decode_inputs(2, 8, 2, 900, d, torch.bfloat16, 45, device="cuda")
    kv_len, q_pos = [900, 411], [899, 410]
    if banded:
        out = atw.decode_banded(q, atw.kcache_band(kc), vc, kv_len, q_pos, rope_base=1e4, k_turns=0.0,
                                num_splits=7, rope_scaling=sc)
    else:
        out = atw.decode(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.0, num_splits=7,
                         rope_scaling=sc)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.0, scaling=sc)
    err = bf16_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert err <= BF16_TOL


def test_prefill_sparse_explicit_widths():
    d = 128
    sc = {"widths": _explicit_widths(d, 46, 500)}
    say("sparse prefill explicit widths d=128")
    q, k, v = synth.prefill_inputs(1, 4, 2, 600, 600, d, torch.bfloat16, 47, device="cuda")
    sel = torch.from_numpy(np.random.default_rng(48).random((1, 4, 10, 10)) < 0.5)
    out = atw.prefill_sparse(q, k, v, atw.pack_block_mask(sel).cuda(), rope_base=1e4, k_turns=0.0,
                             rope_scaling=sc)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, 0.0, scaling=sc, key_blocks=sel.numpy())
    err = bf16_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(to_np(out)).all() and err <= BF16_TOL


@pytest.mark.parametrize("banded", [False, True])
def test_decode_multi_explicit_widths(banded):
    """Draft tokens with an explicit window table: windows that end between
    the tokens' distances (the per-token recomputation) come from the table."""
    d, B, T, hq, hkv, L = 128, 2, 4, 6, 2, 700
    sc = {"widths": _explicit_widths(d, 49, 700)}
    say(f"decode multi explicit widths banded={banded}")
    q = torch.randn((B, T, hq, d), generator=synth.generator(50)).to(torch.bfloat16).cuda()
    _, kc, vc = synth.decode_inputs(B, hq, hkv, L, d, torch.bfloat16, 51, device="cuda")
    kv_len, q_pos = [700, 404], [700 - T, 404 - T]
    kk = atw.kcache_band(kc) if banded else kc
    out = atw.decode_multi(q, kk, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.0, num_splits=7,
                           k_banded=banded, rope_scaling=sc)
    sync()
    ref = oracle.decode_multi(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.0, scaling=sc)
    err = bf16_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(to_np(out)).all() and err <= BF16_TOL
