"""Host-side tests of libatw (no GPU needed): the library loads, exports every
symbol include/atw.h declares, and its planner matches the oracle bit-exactly
(integer windows, pruned/total counts, tile plans); invalid arguments return
the documented codes before any launch."""

import ctypes
import math
import os
import re

import numpy as np
import pytest
import torch

import oracle
import rope_frequency_pair_amd as atw
from rope_frequency_pair_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(atw.LIB_PATH):
        pytest.skip("libatw.so not built (run __graft_entry__.build())")
    return atw.load_library()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "atw.h")).read()
    declared = set(re.findall(r"\b(atw_[a-z_]+)\s*\(", header))
    assert declared == set(binding.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in atw.version()


WINDOW_CASES = [(64, 1e4, 4.0), (64, 1e6, 8.0), (128, 5e5, 8.0), (128, 1e7, 8.0), (128, 1e7, 64.0),
                (2, 10.0, 0.5), (16, 50.0, 1.0), (256, 1e4, 3.0), (96, 123456.0, 0.37)]


@pytest.mark.parametrize("d,base,k", WINDOW_CASES)
def test_widths_bit_exact(lib, d, base, k):
    assert atw.window_widths(d, base, k, True) == list(oracle.window_widths(d, base, k, True))
    assert atw.window_widths(d, base, k, False) == [atw.UNBOUNDED] * (d // 2)
    assert atw.window_widths(d, base, math.inf, True) == [atw.UNBOUNDED] * (d // 2)


def test_widths_random_grid_bit_exact(lib):
    rng = np.random.default_rng(3)
    for _ in range(300):
        d = int(rng.choice([2, 8, 32, 64, 128, 256]))
        base = float(10 ** rng.uniform(0.5, 9))
        k = float(10 ** rng.uniform(-2, 3))
        assert atw.window_widths(d, base, k) == list(oracle.window_widths(d, base, k)), (d, base, k)


def test_counts_bit_exact_small(lib):
    rng = np.random.default_rng(5)
    for _ in range(200):
        d = int(rng.choice([2, 4, 8, 16, 64]))
        base = float(rng.choice([3.0, 10.0, 100.0, 1e4]))
        k = float(rng.choice([0.01, 0.2, 0.5, 1.0, 3.0]))
        n_q, n_kv, p0 = int(rng.integers(0, 50)), int(rng.integers(0, 90)), int(rng.integers(0, 70))
        causal, on = bool(rng.integers(0, 2)), bool(rng.integers(0, 4))
        got = atw.pruned_terms(n_q, n_kv, p0, d, base, k, causal, on)
        assert got == oracle.pruned_terms_bruteforce(n_q, n_kv, p0, d, base, k, causal, on)


@pytest.mark.parametrize("n_q,n_kv,p0,d,base,k", [
    (1024, 1024, 0, 64, 1e4, 4.0),
    (32768, 32768, 0, 64, 1e6, 8.0),
    (131072, 131072, 0, 128, 5e5, 8.0),
    (1, 524288, 524288, 128, 1e7, 8.0),          # the decode row: query at L, keys 0..L-1
    (65536, 1048576, 983040, 128, 1e7, 64.0),    # last 64K chunk of the 1M request
    (1048576, 1048576, 0, 128, 1e7, 64.0),
])
def test_counts_bit_exact_workloads(lib, n_q, n_kv, p0, d, base, k):
    for causal in (True, False):
        got = atw.pruned_terms(n_q, n_kv, p0, d, base, k, causal, True)
        assert got == oracle.pruned_terms(n_q, n_kv, p0, d, base, k, causal, True)


def test_workload_count_values(lib):
    # exact per-head counts of the five workloads (the square ones also equal
    # the per-pair series of the oracle)
    assert atw.pruned_terms(1024, 1024, 0, 64, 1e4, 4.0) == \
        oracle.pruned_terms_square_closed_form(1024, 64, 1e4, 4.0)
    p, t = atw.pruned_terms(131072, 131072, 0, 128, 5e5, 8.0)
    assert (p, t) == oracle.pruned_terms_square_closed_form(131072, 128, 5e5, 8.0)
    assert abs(p / t - 0.4930) < 1e-4
    # 1M request = sum of its 16 chunks
    tot_p = tot_t = 0
    for c in range(16):
        pp, tt = atw.pruned_terms(65536, 65536 * (c + 1), 65536 * c, 128, 1e7, 64.0)
        tot_p += pp
        tot_t += tt
    assert (tot_p, tot_t) == oracle.pruned_terms_square_closed_form(1048576, 128, 1e7, 64.0)


@pytest.mark.parametrize("n_q,n_kv,p0,causal,tq,tk", [
    (300, 300, 0, True, 32, 64), (256, 1000, 744, True, 32, 64), (77, 200, 0, False, 16, 64),
    (1024, 1024, 0, True, 256, 64), (33, 33, 5, True, 7, 9),
])
def test_tile_plan_bit_exact(lib, n_q, n_kv, p0, causal, tq, tk):
    for d, base, k in [(64, 1e4, 4.0), (16, 100.0, 0.7), (128, 5e5, 0.1)]:
        w = oracle.window_widths(d, base, k)
        ref = oracle.tile_plan(n_q, n_kv, p0, causal, tq, tk, w)
        got = np.array(atw.window_plan(d, base, k, True, n_q, n_kv, p0, causal, tq, tk), dtype=np.int32)
        np.testing.assert_array_equal(got.reshape(ref.shape), ref)


def test_invalid_arguments(lib):
    c64 = ctypes.c_int64
    p, t = c64(), c64()
    # head_dim odd, base <= 1, k <= 0 with window on
    assert lib.atw_pruned_terms(10, 10, 0, 63, 1e4, 4.0, 1, 1, ctypes.byref(p), ctypes.byref(t)) == atw.binding.ATW_EINVAL
    assert lib.atw_pruned_terms(10, 10, 0, 64, 1.0, 4.0, 1, 1, ctypes.byref(p), ctypes.byref(t)) == atw.binding.ATW_EINVAL
    assert lib.atw_pruned_terms(10, 10, 0, 64, 1e4, 0.0, 1, 1, ctypes.byref(p), ctypes.byref(t)) == atw.binding.ATW_EINVAL
    assert b"k_turns" in lib.atw_last_error()
    # k ignored when the window is off
    assert lib.atw_pruned_terms(10, 10, 0, 64, 1e4, 0.0, 1, 0, ctypes.byref(p), ctypes.byref(t)) == 0
    assert p.value == 0 and t.value == 32 * 55
    # prefill argument errors are reported before touching any pointer
    s = binding._arr64([0, 0, 0])
    fake = ctypes.c_void_p(16)
    args = dict(dtype=1, batch=1, n_q=10, n_kv=10, q_pos0=0, h_q=4, h_kv=2, d=128)

    def pre(**kw):
        a = dict(args, **kw)
        return lib.atw_prefill(fake, fake, fake, fake, a["dtype"], a["batch"], a["n_q"], a["n_kv"],
                               a["q_pos0"], a["h_q"], a["h_kv"], None, a["d"], s, s, s, s, 1e4, 4.0, 1,
                               1, 0.0, fake, a.get("ws", 1 << 40), None)

    assert pre(d=96) == atw.binding.ATW_EUNSUPPORTED
    assert pre(dtype=7) == atw.binding.ATW_EUNSUPPORTED
    assert pre(h_q=3) == atw.binding.ATW_EINVAL
    assert pre(n_kv=0) == atw.binding.ATW_EINVAL
    assert pre(batch=0) == atw.binding.ATW_EINVAL
    assert lib.atw_prefill(None, fake, fake, fake, 1, 1, 10, 10, 0, 4, 2, None, 128, s, s, s, s, 1e4,
                           4.0, 1, 1, 0.0, fake, 1 << 40, None) == atw.binding.ATW_EINVAL
    bad = binding._arr64([0, 0, 3])   # 3 bf16 elements = 6 bytes: not 16-byte multiple
    assert lib.atw_prefill(fake, fake, fake, fake, 1, 1, 10, 10, 0, 4, 2, None, 128, bad, s, s, s, 1e4,
                           4.0, 1, 1, 0.0, fake, 1 << 40, None) == atw.binding.ATW_EUNSUPPORTED
    hmap = binding._arr32([0, 1, 2, 0])  # kv head 2 does not exist
    assert lib.atw_prefill(fake, fake, fake, fake, 1, 1, 10, 10, 0, 4, 2, hmap, 128, s, s, s, s, 1e4,
                           4.0, 1, 1, 0.0, fake, 1 << 40, None) == atw.binding.ATW_EINVAL
    # workspace: bf16 needs one packed copy of K and V (64-key tiles) and the
    # range maxima (32 chunks x 2 words per (batch, kv head)), fp32 none
    need = lib.atw_prefill_workspace_bytes(1, 1, 2, 10, 128)
    assert need == 2 * 1 * 2 * 1 * 64 * 128 * 2 + 1 * 2 * 32 * 2 * 4
    assert lib.atw_prefill_workspace_bytes(0, 1, 2, 10, 128) == 0
    assert lib.atw_prefill_workspace_bytes(atw.binding.ATW_BF16_F32OUT, 1, 2, 10, 128) == need
    assert pre(ws=need - 1) == atw.binding.ATW_EWORKSPACE


def test_decode_invalid_arguments(lib):
    s3, s2 = binding._arr64([0, 0, 0]), binding._arr64([0, 0])
    fake = ctypes.c_void_p(16)
    kv, qp = binding._arr64([100]), binding._arr64([99])
    need = lib.atw_decode_workspace_bytes(1, 4, 128, 8)
    assert need == 4 * 8 * (128 + 4) * 4

    def dec(kv=kv, qp=qp, ws=need, causal=1, splits=8, dtype=1):
        return lib.atw_decode(fake, fake, fake, fake, dtype, 1, kv, qp, 4, 2, None, 128, s2, s3, s3, s2,
                              1e4, 4.0, causal, 1, 0.0, splits, fake, ws, None)

    assert dec(ws=need - 1) == atw.binding.ATW_EWORKSPACE
    assert dec(qp=binding._arr64([50])) == atw.binding.ATW_EINVAL      # causal needs q_pos >= kv_len-1
    assert dec(kv=binding._arr64([0])) == atw.binding.ATW_EINVAL
    assert dec(splits=0) == atw.binding.ATW_EINVAL
    assert dec(dtype=0) == atw.binding.ATW_EUNSUPPORTED
    assert dec(dtype=3) == atw.binding.ATW_EUNSUPPORTED
    # bf16 inputs with an fp32 output validate like bf16 (the workspace check
    # is reached)
    assert dec(dtype=atw.binding.ATW_BF16_F32OUT, ws=need - 1) == atw.binding.ATW_EWORKSPACE
    # the banded entry point validates the same way
    assert lib.atw_decode_banded(fake, fake, fake, fake, 1, 1, kv, qp, 4, 2, None, 128, s2, s3, s3,
                                 s2, 1e4, 4.0, 1, 1, 0.0, 8, fake, need - 1,
                                 None) == atw.binding.ATW_EWORKSPACE


def test_kcache_band_invalid_arguments(lib):
    s3 = binding._arr64([0, 0, 0])
    fake = ctypes.c_void_p(16)

    def band(d=128, dtype=1, t0=0, n=10, rows=fake, strides=s3):
        return lib.atw_kcache_band(rows, fake, dtype, 1, 2, d, t0, n, strides, s3, None)

    assert band(d=96) == atw.binding.ATW_EUNSUPPORTED
    assert band(dtype=0) == atw.binding.ATW_EUNSUPPORTED
    assert band(t0=-1) == atw.binding.ATW_EINVAL
    assert band(t0=1 << 30) == atw.binding.ATW_EINVAL
    assert band(rows=None) == atw.binding.ATW_EINVAL
    assert band(strides=binding._arr64([0, 0, 3])) == atw.binding.ATW_EUNSUPPORTED
    assert band(n=0, rows=None) == atw.binding.ATW_OK        # nothing to copy, nothing launched


LLAMA32 = {"rope_type": "llama3", "factor": 32.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
           "original_max_position_embeddings": 8192}
SCALINGS = [LLAMA32, dict(LLAMA32, factor=8.0), {"rope_type": "linear", "factor": 4.0},
            {"rope_type": "linear", "factor": 1.0}]


@pytest.mark.parametrize("sc", SCALINGS)
def test_rope_scaling_widths_and_counts_bit_exact(lib, sc):
    for d, base, k in ((128, 5e5, 8.0), (64, 1e6, 8.0), (128, 1e7, 64.0), (64, 1e4, 0.7)):
        assert atw.window_widths(d, base, k, True, sc) == list(oracle.window_widths(d, base, k, True, sc))
        theta = atw.rope_theta(d, base, sc)
        assert np.allclose(theta, oracle.pair_frequencies(d, base, sc), rtol=4e-16, atol=0)
        for n, q0 in ((1000, 0), (4097, 123), (131072, 0)):
            assert atw.pruned_terms(n, n + q0, q0, d, base, k, True, True, sc) == \
                oracle.pruned_terms(n, n + q0, q0, d, base, k, True, True, sc)


def test_rope_table_and_plain_descriptor_match_plain(lib):
    d, base = 128, 5e5
    tab = {"rope_type": "table", "theta": atw.rope_theta(d, base)}
    assert atw.window_widths(d, base, 8.0, True, tab) == atw.window_widths(d, base, 8.0, True)
    assert atw.pruned_terms(5000, 5000, 0, d, None, 8.0, True, True, tab) == \
        atw.pruned_terms(5000, 5000, 0, d, base, 8.0, True, True)


@pytest.mark.parametrize("bad", [
    {"rope_type": "table", "theta": [1.0, 0.5, 0.6, 0.1]},        # rising
    {"rope_type": "table", "theta": [1.0, 0.5, 0.0, 0.0]},        # zero
    {"rope_type": "table", "theta": [1.0, float("nan"), 0.1, 0.01]},
    {"rope_type": "linear", "factor": 0.0},
    {"rope_type": "linear", "factor": -2.0},
    dict(LLAMA32, high_freq_factor=1.0),                          # high <= low
    dict(LLAMA32, original_max_position_embeddings=0),
])
def test_rope_scaling_rejected(lib, bad):
    with pytest.raises(atw.AtwError) as e:
        atw.window_widths(8, 1e4, 1.0, True, bad)
    assert e.value.code == binding.ATW_EINVAL


def _explicit(d, seed):
    """A non-decreasing window table with zeros, short windows and unbounded
    pairs, not of the form floor(k * lambda_r)."""
    rng = np.random.default_rng(seed)
    h = d // 2
    w = np.sort(rng.integers(0, 5000, h))
    w[: h // 8] = 0
    w[h - h // 8:] = 1 << 62
    return [int(x) for x in w]


@pytest.mark.parametrize("kind", [None, "llama3", "linear"])
def test_explicit_widths_used_as_given(lib, kind):
    for d in (64, 128):
        table = _explicit(d, d)
        sc = {"widths": table}
        if kind == "llama3":
            sc = dict(LLAMA32, widths=table)
        elif kind == "linear":
            sc = {"rope_type": "linear", "factor": 4.0, "widths": table}
        for k in (8.0, 0.0, -1.0):       # k is not used with a table
            assert atw.window_widths(d, 5e5, k, True, sc) == table
            assert atw.window_widths(d, 5e5, k, True, sc) == list(oracle.window_widths(d, 5e5, k, True, sc))
        # the frequencies (the rotation) are still the descriptor's
        assert atw.rope_theta(d, 5e5, sc) == atw.rope_theta(d, 5e5, None if kind is None else
                                                               {kk: vv for kk, vv in sc.items() if kk != "widths"})
        assert atw.window_widths(d, 5e5, 8.0, False, sc) == [1 << 62] * (d // 2)
        for n, q0 in ((1000, 0), (4097, 123), (131072, 0)):
            for causal in (True, False):
                assert atw.pruned_terms(n, n + q0, q0, d, 5e5, 1.0, causal, True, sc) == \
                    oracle.pruned_terms(n, n + q0, q0, d, 5e5, 1.0, causal, True, sc)


def test_explicit_widths_clamped_and_counts_sparse(lib):
    d = 64
    table = [0] * 8 + [3, 3, 64, 65, 200, 1000, 4096] + [9000] * 9 + [(1 << 63) - 1] * 8
    sc = {"widths": table}
    assert atw.window_widths(d, 1e4, 1.0, True, sc) == [min(x, 1 << 62) for x in table]
    rng = np.random.default_rng(5)
    n_q, n_kv, q0 = 700, 900, 200
    sel = rng.random((-(-n_q // 64), -(-n_kv // 64))) < 0.4
    packed = atw.pack_block_mask(torch.from_numpy(sel))
    got = atw.pruned_terms_sparse(n_q, n_kv, q0, d, 1e4, 1.0, packed, True, True, sc)
    ref = oracle.pruned_terms_blocks(n_q, n_kv, q0, d, 1e4, 1.0, sel, True, True, sc)
    assert tuple(got) == tuple(ref)


@pytest.mark.parametrize("bad", [[0, 1, 2, -1], [5, 4, 6, 7], [0, 0, 10, 9]])
def test_explicit_widths_rejected(lib, bad):
    with pytest.raises(atw.AtwError) as e:
        atw.window_widths(8, 1e4, 1.0, True, {"widths": bad})
    assert e.value.code == binding.ATW_EINVAL
    with pytest.raises(ValueError):
        atw.window_widths(8, 1e4, 1.0, True, {"widths": [0, 1, 2]})     # wrong length


def _packed_rows(sel):
    """Pack a boolean [n_qb, n_kb] block selection into uint32 words (LSB first)."""
    n_qb, n_kb = sel.shape
    words = -(-n_kb // 32)
    out = np.zeros((n_qb, words), dtype=np.uint32)
    for kb in range(n_kb):
        out[:, kb // 32] |= sel[:, kb].astype(np.uint32) << np.uint32(kb % 32)
    return out


@pytest.mark.parametrize("n_q,n_kv,q_pos0,causal,d,base,k", [
    (700, 700, 0, True, 64, 1e4, 2.0), (300, 2100, 1800, True, 128, 5e5, 8.0),
    (257, 3000, 0, False, 64, 1e6, 0.5), (64 * 40, 64 * 40, 0, True, 128, 1e7, 8.0),
    (1, 5000, 4999, True, 128, 1e7, 8.0)])
def test_sparse_counts_bit_exact(lib, n_q, n_kv, q_pos0, causal, d, base, k):
    n_qb, n_kb = -(-n_q // 64), -(-n_kv // 64)
    sel = np.random.default_rng(n_q + n_kv).random((n_qb, n_kb)) < 0.35
    packed = _packed_rows(sel)
    assert packed.shape[1] == lib.atw_block_mask_words(n_kv)
    c64 = ctypes.c_int64
    p, t = c64(), c64()
    r = binding.rope_descriptor(base, None, d)
    assert lib.atw_pruned_terms_sparse(n_q, n_kv, q_pos0, d, ctypes.byref(r), k, int(causal), 1,
                                       packed.ctypes.data_as(ctypes.c_void_p), ctypes.byref(p),
                                       ctypes.byref(t)) == 0
    assert (p.value, t.value) == oracle.pruned_terms_blocks(n_q, n_kv, q_pos0, d, base, k, sel, causal)
    # the torch packing helper gives the same words
    import torch
    words = atw.pack_block_mask(torch.tensor(sel)).numpy().view(np.uint32)
    assert np.array_equal(words, packed)
    # every block selected: the dense count
    full = _packed_rows(np.ones((n_qb, n_kb), dtype=bool))
    assert lib.atw_pruned_terms_sparse(n_q, n_kv, q_pos0, d, ctypes.byref(r), k, int(causal), 1,
                                       full.ctypes.data_as(ctypes.c_void_p), ctypes.byref(p),
                                       ctypes.byref(t)) == 0
    assert (p.value, t.value) == atw.pruned_terms(n_q, n_kv, q_pos0, d, base, k, causal)


def test_sparse_invalid_arguments(lib):
    s = binding._arr64([0, 0, 0])
    fake = ctypes.c_void_p(16)
    r = binding.rope_descriptor(1e4, None, 128)

    def pre(dtype=1, mask=fake, d=128):
        return lib.atw_prefill_sparse(fake, fake, fake, fake, dtype, 1, 10, 10, 0, 4, 2, None, d, s, s, s,
                                      s, ctypes.byref(r), 4.0, 1, 1, 0.0, mask, fake, 1 << 40, None)

    assert pre(dtype=0) == atw.binding.ATW_EUNSUPPORTED        # fp32: dense path only
    assert pre(mask=None) == atw.binding.ATW_EINVAL
    assert pre(mask=ctypes.c_void_p(18)) == atw.binding.ATW_EINVAL
    assert pre(d=96) == atw.binding.ATW_EUNSUPPORTED
    assert lib.atw_block_mask_words(0) == 0 and lib.atw_block_mask_words(64 * 32) == 1
    assert lib.atw_block_mask_words(64 * 32 + 1) == 2
    p, t = ctypes.c_int64(), ctypes.c_int64()
    assert lib.atw_pruned_terms_sparse(10, 10, 0, 64, ctypes.byref(r), 4.0, 1, 1, None, ctypes.byref(p),
                                       ctypes.byref(t)) == atw.binding.ATW_EINVAL


def test_decode_sparse_invalid_arguments(lib):
    s3, s2 = binding._arr64([0, 0, 0]), binding._arr64([0, 0])
    fake = ctypes.c_void_p(16)
    r = binding.rope_descriptor(1e4, None, 128)
    kv = binding._arr64([5000])
    qp = binding._arr64([4999])

    def dec(mask=fake, words=3, banded=0):
        return lib.atw_decode_sparse(fake, fake, fake, fake, 1, 1, kv, qp, 4, 2, None, 128, s2, s3, s3, s2,
                                     ctypes.byref(r), 4.0, 1, 1, 0.0, 8, mask, words, banded, fake, 1 << 30,
                                     None)

    assert lib.atw_block_mask_words(5000) == 3
    assert dec(mask=None) == atw.binding.ATW_EINVAL
    assert dec(mask=ctypes.c_void_p(18)) == atw.binding.ATW_EINVAL
    assert dec(words=2) == atw.binding.ATW_EINVAL
    assert b"mask_words" in lib.atw_last_error()


def test_rope_flags_contract(lib):
    """atw_rope.flags: widths is read only under ATW_ROPE_HAS_WIDTHS (a caller
    of the 0.1 layout, whose word here was a reserved 0, never has a stale
    pointer read); the flag with a NULL table and unknown bits are rejected."""
    d = 8
    out = (ctypes.c_int64 * (d // 2))()
    plain = atw.window_widths(d, 1e4, 1.0, True)
    r = binding.Rope()
    r.kind = binding.ATW_ROPE_PLAIN
    r.base = 1e4
    table = (ctypes.c_int64 * (d // 2))(0, 1, 2, 3)
    r.widths = ctypes.cast(table, ctypes.POINTER(ctypes.c_int64))
    # flag clear: the pointer is ignored, windows come from k
    assert lib.atw_window_widths_rope(ctypes.byref(r), d, 1.0, 1, out) == binding.ATW_OK
    assert list(out) == plain
    r.flags = binding.ATW_ROPE_HAS_WIDTHS
    assert lib.atw_window_widths_rope(ctypes.byref(r), d, 1.0, 1, out) == binding.ATW_OK
    assert list(out) == [0, 1, 2, 3]
    r.widths = ctypes.cast(None, ctypes.POINTER(ctypes.c_int64))
    assert lib.atw_window_widths_rope(ctypes.byref(r), d, 1.0, 1, out) == binding.ATW_EINVAL
    r.widths = ctypes.cast(table, ctypes.POINTER(ctypes.c_int64))
    for bad in (2, 4, -1):
        r.flags = bad
        assert lib.atw_window_widths_rope(ctypes.byref(r), d, 1.0, 1, out) == binding.ATW_EINVAL
