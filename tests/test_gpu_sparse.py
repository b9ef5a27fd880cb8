"""GPU parity of the block-sparse composition (atw_prefill_sparse): a
token-level block selection decides which keys a query attends and the
per-pair window applies on top of it ("ATFlash: Per-RoPE-Wavelength Attention
Windows for Compute/Memory-Efficient LLM Inference", arXiv abstract).  Checked
against the fp64 oracle with the same selection: whole outputs at sizes with
several workgroups, key tiles and a ragged tail, query blocks that attend
nothing, a chunk (q_pos0 > 0), non-causal, rescaled frequencies, and sampled
rows at the 128K Llama-3.2-3B shape; and bit-identity with the dense path
when every block is selected."""

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import synth
from tests.gpu_util import BF16_TOL, bf16_err, check_rows, max_err, sample_rows, say, sync, to_np

pytestmark = pytest.mark.gpu

SMALL_LLAMA3 = {"rope_type": "llama3", "factor": 4.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                "original_max_position_embeddings": 256}


def _random_selection(batch, h_q, n_q, n_kv, seed, density, empty_block=None):
    n_qb, n_kb = -(-n_q // 64), -(-n_kv // 64)
    sel = torch.from_numpy(np.random.default_rng(seed).random((batch, h_q, n_qb, n_kb)) < density)
    if empty_block is not None and empty_block < n_qb:
        sel[:, :, empty_block] = False
    return sel


CASES = [
    # d, h_q, h_kv, n_q, n_kv, q_pos0, causal, k_turns, density
    (128, 6, 2, 700, 700, 0, True, 0.5, 0.35),
    (64, 7, 1, 1000, 1000, 0, True, 2.0, 0.3),
    (128, 4, 4, 300, 900, 600, True, 1.0, 0.5),
    (64, 4, 2, 500, 530, 0, False, 1.0, 0.4),
]


@pytest.mark.parametrize("d,h_q,h_kv,n_q,n_kv,q_pos0,causal,k_turns,density", CASES)
def test_sparse_prefill_parity(d, h_q, h_kv, n_q, n_kv, q_pos0, causal, k_turns, density):
    say(f"sparse prefill d={d} heads {h_q}/{h_kv} n_q={n_q} n_kv={n_kv} q_pos0={q_pos0} causal={causal}")
    q, k, v = synth.prefill_inputs(2, h_q, h_kv, n_q, n_kv, d, torch.bfloat16, 60 + d, device="cuda")
    sel = _random_selection(2, h_q, n_q, n_kv, 61 + n_q, density, empty_block=2)
    mask = atw.pack_block_mask(sel).cuda()
    ref_args = (to_np(q), to_np(k), to_np(v), q_pos0, 1e4, k_turns)
    for window_on in (True, False):
        out = atw.prefill_sparse(q, k, v, mask, rope_base=1e4, k_turns=k_turns, q_pos0=q_pos0,
                                 causal=causal, window_on=window_on)
        sync()
        ref = oracle.prefill(*ref_args, causal=causal, window_on=window_on, key_blocks=sel.numpy())
        got = to_np(out)
        err = bf16_err(got, ref)
        say(f"  window_on={window_on} max abs err {err:.3e}")
        assert np.isfinite(got).all() and err <= BF16_TOL
        # a query block that attends nothing gives exactly 0
        assert np.all(got[:, :, 128:192] == 0.0)


@pytest.mark.parametrize("d", [64, 128])
def test_all_blocks_selected_is_dense_bitwise(d):
    say(f"sparse all-selected == dense, d={d}")
    q, k, v = synth.prefill_inputs(1, 4, 2, 900, 900, d, torch.bfloat16, 62, device="cuda")
    sel = torch.ones((1, 4, -(-900 // 64), -(-900 // 64)), dtype=torch.bool)
    mask = atw.pack_block_mask(sel).cuda()
    for k_turns in (0.3, 4.0):
        a = atw.prefill_sparse(q, k, v, mask, rope_base=1e4, k_turns=k_turns)
        b = atw.prefill(q, k, v, rope_base=1e4, k_turns=k_turns)
        sync()
        assert torch.equal(a, b)


def test_sparse_prefill_rope_scaling():
    say("sparse prefill with llama3 rope scaling")
    q, k, v = synth.prefill_inputs(1, 4, 2, 600, 600, 128, torch.bfloat16, 63, device="cuda")
    sel = synth.block_selection(1, 4, 600, 600, 64, density=0.3, local=2)
    mask = atw.pack_block_mask(sel).cuda()
    out = atw.prefill_sparse(q, k, v, mask, rope_base=1e4, k_turns=0.6, rope_scaling=SMALL_LLAMA3)
    sync()
    ref = oracle.prefill(to_np(q), to_np(k), to_np(v), 0, 1e4, 0.6, scaling=SMALL_LLAMA3,
                         key_blocks=sel.numpy())
    err = bf16_err(to_np(out), ref)
    say(f"  max abs err {err:.3e}")
    assert err <= BF16_TOL


def test_sparse_llama_128k_sampled_rows():
    """The benchmark's 128K block-sparse workload (sink + local band + 10% of
    earlier blocks), sampled rows of two heads against the oracle."""
    w = synth.WORKLOADS["llama-3.2-3b-128k"]
    say("sparse 128k: inputs and selection")
    q, k, v = synth.workload_prefill_inputs(w)
    sel = synth.block_selection(w.batch, w.h_q, w.n, w.n, w.seed + 100)
    mask = atw.pack_block_mask(sel).cuda()
    say("sparse 128k: running")
    out = atw.prefill_sparse(q, k, v, mask, rope_base=w.rope_base, k_turns=w.k_turns)
    sync()
    heads = [0, 23]
    G = w.h_q // w.h_kv
    kvs = sorted({h // G for h in heads})
    hmap = [kvs.index(h // G) for h in heads]
    rows = sample_rows(w.n, seed=w.seed, count=3)
    qn = to_np(q[:, heads][:, :, rows])
    kn, vn = to_np(k[:, kvs]), to_np(v[:, kvs])
    seln = sel[:, heads].numpy()
    say(f"sparse 128k: oracle on {len(rows)} rows x {len(heads)} heads")
    ref = np.zeros((1, len(heads), len(rows), w.head_dim))
    for i, r in enumerate(rows):
        n_kb = r // 64 + 1
        kb_row = seln[:, :, r // 64:r // 64 + 1, :n_kb]
        ref[:, :, i] = oracle.prefill(qn[:, :, i:i + 1], kn[:, :, :r + 1], vn[:, :, :r + 1], r,
                                      w.rope_base, w.k_turns, kv_head_of_q=hmap,
                                      key_blocks=kb_row)[:, :, 0]
    check_rows(to_np(out[:, heads][:, :, rows]), ref, "sparse 128k")


@pytest.mark.parametrize("splits", [7, 64])
@pytest.mark.parametrize("banded", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_sparse_decode_parity(d, banded, splits):
    say(f"sparse decode d={d} banded={banded} splits={splits}")
    kv_len = [3000, 1777, 64]
    q, kc, vc = synth.decode_inputs(3, 8, 2, 3000, d, torch.bfloat16, 70 + d, device="cuda")
    sel = synth.decode_block_selection(3, 2, kv_len, 71, density=0.3, local=2)
    sel[1, 1] = False                      # a (sequence, kv head) that attends nothing
    mask = atw.pack_block_mask(sel).cuda()
    kin = atw.kcache_band(kc) if banded else kc
    for window_on, k_turns in ((True, 0.7), (True, 4.0), (False, 1.0)):
        out = atw.decode_sparse(q, kin, vc, kv_len, [n - 1 for n in kv_len], mask, rope_base=1e4,
                                k_turns=k_turns, window_on=window_on, num_splits=splits, k_banded=banded)
        sync()
        ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, [n - 1 for n in kv_len], 1e4, k_turns,
                            window_on=window_on, key_blocks=sel.numpy())
        got = to_np(out)
        err = bf16_err(got, ref)
        say(f"  window_on={window_on} k={k_turns} max abs err {err:.3e}")
        assert np.isfinite(got).all() and err <= BF16_TOL
        assert np.all(got[1, 4:] == 0.0)


def test_sparse_decode_all_selected_matches_dense():
    """Every block selected: the dense decode's result (within rounding: the
    split partition differs)."""
    q, kc, vc = synth.decode_inputs(2, 14, 2, 2500, 128, torch.bfloat16, 72, device="cuda")
    sel = torch.ones((2, 2, -(-2500 // 64)), dtype=torch.bool)
    mask = atw.pack_block_mask(sel).cuda()
    a = atw.decode_sparse(q, kc, vc, [2500, 900], [2499, 899], mask, rope_base=1e6, k_turns=2.0, num_splits=16)
    b = atw.decode(q, kc, vc, [2500, 900], [2499, 899], rope_base=1e6, k_turns=2.0, num_splits=16)
    sync()
    assert max_err(to_np(a), to_np(b).astype(np.float64)) <= BF16_TOL


def test_sparse_decode_workload_512k_sampled():
    """The 512K decode workload with a page-level selection (first block, last
    four blocks, 5% of the rest per (sequence, kv head)), banded K cache."""
    w = synth.WORKLOADS["qwen2.5-7b-1m-decode-512k"]
    say("sparse decode 512k: inputs")
    q, kc, vc = synth.workload_decode_inputs(w)
    L = w.n
    sel = synth.decode_block_selection(w.batch, w.h_kv, L, w.seed + 100)
    mask = atw.pack_block_mask(sel).cuda()
    kb = atw.kcache_band(kc)
    say("sparse decode 512k: running")
    out = atw.decode_sparse(q, kb, vc, [L] * w.batch, [L] * w.batch, mask, rope_base=w.rope_base,
                            k_turns=w.k_turns, num_splits=w.splits, k_banded=True)
    sync()
    del kb
    G = w.h_q // w.h_kv
    for b, kvh in ((0, 0), (5, 3)):
        heads = list(range(kvh * G, (kvh + 1) * G))
        qn = to_np(q[b:b + 1, heads])
        kn, vn = to_np(kc[b:b + 1, kvh:kvh + 1]), to_np(vc[b:b + 1, kvh:kvh + 1])
        say(f"sparse decode 512k: oracle b={b} kv={kvh}")
        ref = oracle.decode(qn, kn, vn, [L], [L], w.rope_base, w.k_turns, kv_head_of_q=[0] * G,
                            key_blocks=sel[b:b + 1, kvh:kvh + 1].numpy())
        check_rows(to_np(out[b:b + 1, heads]), ref, f"b={b} kv={kvh}")


@pytest.mark.parametrize("banded", [False, True])
def test_sparse_decode_far_apart_blocks(banded):
    """A selection of a few blocks thousands of blocks apart (one split walks
    past 64 mask words between two of them, so it reloads the words it holds),
    against the oracle; sequences with different selections and lengths."""
    L = 300_000                                  # 4688 blocks, 147 mask words
    q, kc, vc = synth.decode_inputs(2, 8, 2, L, 128, torch.bfloat16, 74, device="cuda")
    n_kb = -(-L // 64)
    sel = torch.zeros((2, 2, n_kb), dtype=torch.bool)
    sel[0, 0, [0, 2000, n_kb - 1]] = True        # words 0, 62, 146
    sel[0, 1, [5, 4600]] = True                  # words 0, 143
    sel[1, 0, [3000]] = True
    sel[1, 1, [1, 4100, 4101]] = True
    kv_len = [L, L - 7000]
    sel[1, :, -(-kv_len[1] // 64):] = False
    mask = atw.pack_block_mask(sel).cuda()
    kin = atw.kcache_band(kc) if banded else kc
    say(f"sparse decode far-apart blocks banded={banded}: oracle")
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), kv_len, [n - 1 for n in kv_len], 1e6, 4.0,
                        key_blocks=sel.numpy())
    for splits in (1, 2, 3):
        out = atw.decode_sparse(q, kin, vc, kv_len, [n - 1 for n in kv_len], mask, rope_base=1e6,
                                k_turns=4.0, num_splits=splits, k_banded=banded)
        sync()
        check_rows(to_np(out), ref, f"splits={splits} banded={banded}")


@pytest.mark.parametrize("banded", [False, True])
def test_sparse_decode_mask_row_past_one_chunk(banded):
    """A mask row longer than the 256 words the split search reads in one
    round trip (over 512K keys): selected blocks on both sides of word 256,
    split starts that fall in the second chunk, against the oracle."""
    L = 700_000                                  # 10938 blocks, 342 mask words
    q, kc, vc = synth.decode_inputs(1, 4, 1, L, 128, torch.bfloat16, 75, device="cuda")
    n_kb = -(-L // 64)
    sel = torch.zeros((1, 1, n_kb), dtype=torch.bool)
    sel[0, 0, [3, 8191, 8192, 8193, 9000, 10500, n_kb - 1]] = True   # words 0, 255, 256, 256, 281, 328, 341
    mask = atw.pack_block_mask(sel).cuda()
    kin = atw.kcache_band(kc) if banded else kc
    say(f"sparse decode mask row past one chunk banded={banded}: oracle")
    ref = oracle.decode(to_np(q), to_np(kc), to_np(vc), [L], [L - 1], 1e6, 4.0, key_blocks=sel.numpy())
    for splits in (1, 2, 3, 5, 7):
        out = atw.decode_sparse(q, kin, vc, [L], [L - 1], mask, rope_base=1e6, k_turns=4.0,
                                num_splits=splits, k_banded=banded)
        sync()
        check_rows(to_np(out), ref, f"splits={splits} banded={banded}")
