"""Randomized prefill parity sweep against the fp64 oracle: head_dim 64/128,
GQA groups 1-8, batch 1-2, ragged query and key counts, chunk offsets
(q_pos0 > 0), keys past the last query, causal and not, windows from
k = 0.01 (almost every pair pruned) to k = 20, rope bases 1e4-1e7, window
off, block selections, fp32 inputs and the fp32-output variant.  Every output
element of every case is compared (sizes the oracle finishes in about a
second); the case parameters are printed before each launch."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import BF16_TOL, F32_TOL, bf16_err, max_err, say, sync, to_np

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(seed)
    d = int(r.choice([64, 128]))
    g = int(r.choice([1, 2, 3, 4, 8]))
    h_kv = int(r.integers(1, 3)) if g <= 4 else 1
    causal = bool(r.random() < 0.8)
    n_q = int(r.integers(1, 501))
    q_pos0 = int(r.choice([0, 0, int(r.integers(1, 800))]))
    if causal:
        n_kv = q_pos0 + n_q + int(r.choice([0, 0, int(r.integers(1, 200))]))
    else:
        n_kv = int(r.integers(1, 801))
    kind = str(r.choice(["bf16", "bf16", "bf16", "f32out", "f32"]))
    return dict(d=d, h_kv=h_kv, h_q=g * h_kv, B=int(r.integers(1, 3)), n_q=n_q, n_kv=n_kv, q_pos0=q_pos0,
                causal=causal, k_turns=float(np.exp(r.uniform(np.log(0.01), np.log(20.0)))),
                base=float(r.choice([1e4, 5e5, 1e6, 1e7])), window_on=bool(r.random() < 0.85), kind=kind,
                sparse=kind != "f32" and bool(r.random() < 0.3), density=float(r.choice([0.1, 0.4, 0.8])))


@pytest.mark.parametrize("seed", range(48))
def test_prefill_random_sweep(seed):
    c = _case(5000 + seed)
    say(f"prefill sweep seed {5000 + seed}: {c}")
    dtype = torch.float32 if c["kind"] == "f32" else torch.bfloat16
    gen = synth.generator(6000 + seed)
    q = torch.randn((c["B"], c["h_q"], c["n_q"], c["d"]), generator=gen).to(dtype).cuda()
    k = torch.randn((c["B"], c["h_kv"], c["n_kv"], c["d"]), generator=gen).to(dtype).cuda()
    v = torch.randn((c["B"], c["h_kv"], c["n_kv"], c["d"]), generator=gen).to(dtype).cuda()
    out = torch.empty(q.shape, dtype=torch.float32 if c["kind"] != "bf16" else torch.bfloat16, device="cuda")
    kw = dict(rope_base=c["base"], k_turns=c["k_turns"], q_pos0=c["q_pos0"], causal=c["causal"],
              window_on=c["window_on"], out=out)
    blocks = None
    if c["sparse"]:
        n_qb, n_kb = -(-c["n_q"] // 64), -(-c["n_kv"] // 64)
        sel = torch.from_numpy(np.random.default_rng(7000 + seed).random((c["B"], c["h_q"], n_qb, n_kb))
                               < c["density"])
        atw.prefill_sparse(q, k, v, atw.pack_block_mask(sel).cuda(), **kw)
        blocks = sel.numpy()
    else:
        atw.prefill(q, k, v, **kw)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), c["q_pos0"], c["base"], c["k_turns"], causal=c["causal"],
                         window_on=c["window_on"], key_blocks=blocks)
    got = to_np(out)
    assert np.isfinite(got).all()
    if c["kind"] == "bf16":
        err, tol = bf16_err(got, ref), BF16_TOL
    else:
        err, tol = max_err(got, ref), (F32_TOL if c["kind"] == "f32" else BF16_TOL)
    say(f"  max abs err {err:.3e} (tol {tol})")
    assert err <= tol, (5000 + seed, err)
