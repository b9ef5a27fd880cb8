"""bf16 inputs with an fp32 output (ATW_BF16_F32OUT): the bf16 path without the
final rounding to bf16.  Its error against the fp64 oracle is the
computation's alone, so the plain 1e-2 bound holds at every output magnitude
(a bf16 output cannot meet it from |o| = 4 on), and rounding the fp32 output
to bf16 gives the bf16 call's output bit for bit.  Every entry point that
takes the element type is covered: prefill (plain, block-sparse, rescaled
frequencies), decode (row and banded cache, draft tokens, block-sparse,
rescaled frequencies, the allocation-free variant)."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import BF16_TOL, max_err, say, sync, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,n,k_turns,seed", [(128, 127, 0.5, 217), (128, 700, 0.35, 7), (64, 700, 4.0, 7),
                                              (64, 255, 0.5, 345)])
def test_prefill_f32_output(d, n, k_turns, seed):
    say(f"prefill bf16 -> f32 d={d} n={n} k={k_turns}")
    hq, hkv = (3, 1) if n in (127, 255) else (4, 2)
    q, k, v = synth.prefill_inputs(1 if n != 700 else 2, hq, hkv, n, n, d, torch.bfloat16, seed, device="cuda")
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns, out=out32)
    out16 = atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, k_turns)
    err = max_err(to_np(out32), ref)
    say(f"  fp32 output: max abs err {err:.3e}; bf16 output: {max_err(to_np(out16), ref):.3e}; "
        f"max |o| {np.abs(ref).max():.2f}")
    assert np.isfinite(to_np(out32)).all() and err <= BF16_TOL
    assert torch.equal(out32.to(torch.bfloat16), out16)


@pytest.mark.parametrize("banded", [False, True])
def test_decode_f32_output(banded):
    say(f"decode bf16 -> f32 banded={banded}")
    q, kc, vc = synth.decode_inputs(3, 8, 2, 1100, 128, torch.bfloat16, 21, device="cuda")
    kv_len, q_pos = [1100, 777, 33], [1099, 826, 32]
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    fn = atw.decode_banded if banded else atw.decode
    kk = atw.kcache_band(kc) if banded else kc
    fn(q, kk, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.5, num_splits=7, out=out32)
    out16 = fn(q, kk, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.5, num_splits=7)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.5)
    err = max_err(to_np(out32), ref)
    say(f"  fp32 output: max abs err {err:.3e}")
    assert np.isfinite(to_np(out32)).all() and err <= BF16_TOL
    assert torch.equal(out32.to(torch.bfloat16), out16)


def test_decode_multi_f32_output():
    say("multi-token decode bf16 -> f32")
    q, kc, vc = synth.decode_inputs(2, 4, 2, 600, 128, torch.bfloat16, 31, device="cuda")
    qm = torch.randn((2, 3, 4, 128), generator=synth.generator(32, "cuda"), device="cuda").to(torch.bfloat16)
    out32 = torch.empty(qm.shape, dtype=torch.float32, device="cuda")
    atw.decode_multi(qm, kc, vc, [600, 500], [597, 497], rope_base=1e4, k_turns=0.5, num_splits=5, out=out32)
    out16 = atw.decode_multi(qm, kc, vc, [600, 500], [597, 497], rope_base=1e4, k_turns=0.5, num_splits=5)
    sync()
    ref = oracle.decode_multi(to_np(qm), to_np(kc), to_np(vc), [600, 500], [597, 497], 1e4, 0.5)
    err = max_err(to_np(out32), ref)
    say(f"  fp32 output: max abs err {err:.3e}")
    assert err <= BF16_TOL
    assert torch.equal(out32.to(torch.bfloat16), out16)


SMALL_LLAMA3 = {"rope_type": "llama3", "factor": 4.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                "original_max_position_embeddings": 256}


def _f32_vs_bf16(out32, out16, ref, label):
    err = max_err(to_np(out32), ref)
    say(f"  {label}: fp32 output max abs err {err:.3e}")
    assert np.isfinite(to_np(out32)).all() and err <= BF16_TOL
    assert torch.equal(out32.to(torch.bfloat16), out16)


@pytest.mark.parametrize("d", [64, 128])
def test_prefill_sparse_f32_output(d):
    say(f"block-sparse prefill bf16 -> f32 d={d}")
    q, k, v = synth.prefill_inputs(2, 6, 2, 700, 700, d, torch.bfloat16, 63, device="cuda")
    sel = torch.from_numpy(np.random.default_rng(64).random((2, 6, 11, 11)) < 0.4)
    mask = atw.pack_block_mask(sel).cuda()
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    atw.prefill_sparse(q, k, v, mask, rope_base=1e4, k_turns=0.5, out=out32)
    out16 = atw.prefill_sparse(q, k, v, mask, rope_base=1e4, k_turns=0.5)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, 0.5, key_blocks=sel.numpy())
    _f32_vs_bf16(out32, out16, ref, "sparse prefill")


def test_prefill_rope_scaling_f32_output():
    say("prefill with llama3 rope scaling bf16 -> f32")
    q, k, v = synth.prefill_inputs(1, 4, 2, 700, 700, 64, torch.bfloat16, 65, device="cuda")
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    atw.prefill(q, k, v, rope_base=1e4, k_turns=0.4, rope_scaling=SMALL_LLAMA3, out=out32)
    out16 = atw.prefill(q, k, v, rope_base=1e4, k_turns=0.4, rope_scaling=SMALL_LLAMA3)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, 0.4, scaling=SMALL_LLAMA3)
    _f32_vs_bf16(out32, out16, ref, "rope-scaled prefill")


@pytest.mark.parametrize("banded", [False, True])
def test_decode_sparse_f32_output(banded):
    say(f"block-sparse decode bf16 -> f32 banded={banded}")
    kv_len = [3000, 1777, 64]
    q_pos = [n - 1 for n in kv_len]
    q, kc, vc = synth.decode_inputs(3, 8, 2, 3000, 128, torch.bfloat16, 66, device="cuda")
    sel = synth.decode_block_selection(3, 2, kv_len, 67, density=0.3, local=2)
    mask = atw.pack_block_mask(sel).cuda()
    kin = atw.kcache_band(kc) if banded else kc
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    atw.decode_sparse(q, kin, vc, kv_len, q_pos, mask, rope_base=1e4, k_turns=0.7, num_splits=7,
                      k_banded=banded, out=out32)
    out16 = atw.decode_sparse(q, kin, vc, kv_len, q_pos, mask, rope_base=1e4, k_turns=0.7, num_splits=7,
                              k_banded=banded)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.7, key_blocks=sel.numpy())
    _f32_vs_bf16(out32, out16, ref, "sparse decode")


def test_decode_rope_scaling_and_noalloc_f32_output():
    say("decode with llama3 rope scaling, and decode_noalloc, bf16 -> f32")
    q, kc, vc = synth.decode_inputs(2, 8, 2, 900, 64, torch.bfloat16, 68, device="cuda")
    kv_len, q_pos = [900, 411], [899, 410]
    out32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    atw.decode(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.6, num_splits=7, rope_scaling=SMALL_LLAMA3,
               out=out32)
    out16 = atw.decode(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.6, num_splits=7,
                       rope_scaling=SMALL_LLAMA3)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.6, scaling=SMALL_LLAMA3)
    _f32_vs_bf16(out32, out16, ref, "rope-scaled decode")
    na32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    atw.decode_noalloc(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.6, num_splits=7, out=na32)
    na16 = atw.decode(q, kc, vc, kv_len, q_pos, rope_base=1e4, k_turns=0.6, num_splits=7)
    sync()
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, q_pos, 1e4, 0.6)
    _f32_vs_bf16(na32, na16, ref, "decode_noalloc")
