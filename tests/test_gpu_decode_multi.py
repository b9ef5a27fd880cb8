"""GPU parity of atw_decode_multi (q_len draft tokens per sequence at
consecutive positions, causal, each with its own window) against the fp64
oracle; consistency with single-token decode; the workload shape of the
Qwen2.5-7B-1M decode with two and four tokens per sequence, sampled."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import BF16_TOL, bf16_err, check_rows, max_err, say, sync, to_np

pytestmark = pytest.mark.gpu


def _inputs(B, T, Hq, Hkv, L, d, seed):
    g = synth.generator(seed)
    q = torch.randn((B, T, Hq, d), generator=g).to(torch.bfloat16).cuda()
    k = torch.randn((B, Hkv, L, d), generator=g).to(torch.bfloat16).cuda()
    v = torch.randn((B, Hkv, L, d), generator=g).to(torch.bfloat16).cuda()
    return q, k, v


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("banded", [False, True])
@pytest.mark.parametrize("T,Hq,Hkv", [(2, 14, 2), (4, 6, 2), (5, 3, 1), (4, 14, 2)])
def test_decode_multi_parity(d, banded, T, Hq, Hkv):
    """Short windows (k = 0.4) put pair windows between the tokens' distances
    in many tiles (the per-token recomputation) and the drafts' own keys are
    masked causally."""
    say(f"decode multi d={d} banded={banded} T={T} heads {Hq}/{Hkv}")
    B, L = 3, 700
    q, kc, vc = _inputs(B, T, Hq, Hkv, L, d, 41 + T)
    kv_len = [700, 404, 37]
    q_pos = [700 - T, 404 - T, 40]     # sequence 2: the tokens sit beyond its cache
    kk = atw.kcache_band(kc) if banded else kc
    for k_turns, splits in ((0.4, 7), (3.0, 64)):
        out = atw.decode_multi(q, kk, vc, kv_len, q_pos, rope_base=1e4, k_turns=k_turns,
                               num_splits=splits, k_banded=banded)
        sync()
        ref = oracle.decode_multi(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, k_turns)
        err = bf16_err(to_np(out), ref)
        say(f"  k={k_turns} splits={splits} max abs err {err:.3e}")
        assert np.isfinite(to_np(out)).all() and err <= BF16_TOL


def test_decode_multi_token_equals_single_decode():
    """Token j equals atw_decode at position q_pos + j over kv_len = q_pos + j + 1."""
    B, T, Hq, Hkv, L, d = 2, 3, 8, 2, 600, 128
    q, kc, vc = _inputs(B, T, Hq, Hkv, L, d, 50)
    q_pos = [597, 300]
    out = atw.decode_multi(q, kc, vc, [600, 303], q_pos, rope_base=1e4, k_turns=0.5, num_splits=5)
    for j in range(T):
        one = atw.decode(q[:, j].contiguous(), kc, vc, [q_pos[0] + j + 1, q_pos[1] + j + 1],
                         [q_pos[0] + j, q_pos[1] + j], rope_base=1e4, k_turns=0.5, num_splits=5)
        sync()
        err = max_err(to_np(out[:, j]), to_np(one).astype(np.float64))
        say(f"  token {j}: max abs diff to single-token decode {err:.3e}")
        assert err <= 4e-3


def test_decode_multi_rope_scaling_and_window_off():
    sc = {"rope_type": "llama3", "factor": 4.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
          "original_max_position_embeddings": 256}
    B, T, Hq, Hkv, L, d = 2, 4, 4, 1, 500, 128
    q, kc, vc = _inputs(B, T, Hq, Hkv, L, d, 51)
    for on in (True, False):
        out = atw.decode_multi(q, kc, vc, [500, 250], [496, 247], rope_base=1e4, k_turns=0.6,
                               window_on=on, num_splits=9, rope_scaling=sc)
        sync()
        ref = oracle.decode_multi(to_np(q), to_np(kc), to_np(vc), [500, 250], [496, 247], 1e4, 0.6,
                                  window_on=on, scaling=sc)
        err = bf16_err(to_np(out), ref)
        say(f"  window_on={on} max abs err {err:.3e}")
        assert err <= BF16_TOL


@pytest.mark.parametrize("T", [2, 4])
def test_decode_multi_workload_512k_sampled(T):
    """Qwen2.5-7B-1M decode shape (28/4 heads, d = 128, base 1e7, k = 8, 64
    splits) at a 512K cache with T draft tokens per sequence; two sequences,
    heads 0 and 27 checked."""
    w = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
    B, L = 2, w.n
    say(f"decode multi 512K T={T}")
    q, kc, vc = _inputs(B, T, w.h_q, w.h_kv, L, w.head_dim, 52 + T)
    q_pos = [L - T, L - T - 1000]
    kv_len = [L, L - 1000]
    out = atw.decode_multi(q, kc, vc, kv_len, q_pos, rope_base=w.rope_base, k_turns=w.k_turns,
                           num_splits=64)
    sync()
    heads = [0, w.h_q - 1]
    kvs = sorted({h // (w.h_q // w.h_kv) for h in heads})
    hmap = [kvs.index(h // (w.h_q // w.h_kv)) for h in heads]
    ref = oracle.decode_multi(to_np(q[:, :, heads]), to_np(kc[:, kvs]), to_np(vc[:, kvs]), kv_len, q_pos,
                              w.rope_base, w.k_turns, kv_head_of_q=hmap)
    check_rows(to_np(out[:, :, heads]), ref, f"T={T}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("banded", [False, True])
def test_decode_multi_every_staging_regime(d, banded):
    """Windows short enough (k = 0.01, 0.05) that, walking from the far keys
    to the near ones, a split passes through tiles where every pair is pruned
    (scores 0), then through tiles that keep only the last 2, 4 and finally
    all pair chunks; one split walks all of them, more splits start inside the
    regimes.  Single-token decode over the same keys (every chunk staged)
    against the oracle too."""
    say(f"decode staging regimes d={d} banded={banded}")
    B, T, Hq, Hkv, L = 2, 3, 6, 2, 3000
    q, kc, vc = _inputs(B, T, Hq, Hkv, L, d, 77)
    kv_len = [3000, 1900]
    q_pos = [3000 - T, 1900 - T]
    kk = atw.kcache_band(kc) if banded else kc
    for k_turns in (0.01, 0.05):
        ref = oracle.decode_multi(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, k_turns)
        ref1 = oracle.decode(to_np(q[:, 0]), to_np(kc), to_np(vc), [p + 1 for p in q_pos], q_pos, 1e4, k_turns)
        for splits in (1, 3, 7):
            out = atw.decode_multi(q, kk, vc, kv_len, q_pos, rope_base=1e4, k_turns=k_turns,
                                   num_splits=splits, k_banded=banded)
            sync()
            check_rows(to_np(out).reshape(-1, d), ref.reshape(-1, d), f"multi k={k_turns} splits={splits}")
            fn = atw.decode_banded if banded else atw.decode
            out1 = fn(q[:, 0].contiguous(), kk, vc, [p + 1 for p in q_pos], q_pos, rope_base=1e4,
                      k_turns=k_turns, num_splits=splits)
            sync()
            check_rows(to_np(out1).reshape(-1, d), ref1.reshape(-1, d), f"single k={k_turns} splits={splits}")
