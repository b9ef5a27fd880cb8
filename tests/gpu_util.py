"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import sys

import numpy as np
import torch

BF16_TOL = 1e-2     # max abs error for bf16 inputs (fp32 accumulation)
F32_TOL = 1e-4      # max abs error for fp32 inputs
# Per-row relative bound for sampled rows deep into long sequences, where the
# outputs are ~1e-3 and the absolute bound alone would accept a zeroed or
# mis-scaled row: max_d |got - ref| <= ROW_REL * max_d |ref| + ROW_ABS.
ROW_REL = 2.0 ** -6
ROW_ABS = 1e-4


def to_np(t):
    """Exact float32 copy of a (bf16 or fp32) tensor as numpy."""
    return t.detach().float().cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_err(got, ref):
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)))


# A bf16 output holds 8 significant bits: at |x| in [2^e, 2^(e+1)) its values
# are 2^(e-7) apart, so the nearest bf16 value to an exact result can be half
# that away -- 7.8e-3 in [2, 4), 1.56e-2 in [4, 8).  From |x| = 4 on, no bf16
# output can meet the 1e-2 bound at every element (the correctly rounded
# exact result misses it by up to 5.6e-3).  Reading of the bound for bf16
# outputs: |got - ref| <= max(BF16_TOL, half_ulp(ref) + BF16_REPR_MARGIN),
# i.e. the computation's error plus the output's own representation error;
# below |ref| = 4 this is the plain 1e-2 bound.
BF16_REPR_MARGIN = 1e-3


def bf16_half_ulp(x):
    """Half the spacing of bf16 values at |x| (largest distance from x to the
    nearest bf16 value)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def bf16_err(got, ref):
    """max_err of a bf16 output against the exact result, less, per element,
    the part of the bound no bf16 value can avoid (zero below |ref| = 4):
    bf16_err(got, ref) <= BF16_TOL  <=>  every element is within
    max(BF16_TOL, half_ulp(ref) + BF16_REPR_MARGIN)."""
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    if err.size == 0:
        return 0.0
    excess = np.maximum(0.0, bf16_half_ulp(ref) + BF16_REPR_MARGIN - BF16_TOL)
    return float(np.max(err - excess))


def row_rel_violation(got, ref, rel=ROW_REL, absolute=ROW_ABS):
    """Largest ratio, over rows (last axis = head dim), of the row's max abs
    error to its bound rel * max|ref_row| + absolute; <= 1 passes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref).max(axis=-1)
    bound = rel * np.abs(ref).max(axis=-1) + absolute
    return float((err / bound).max())


def check_rows(got, ref, label="", tol=BF16_TOL):
    """The parity bar for sampled rows: max abs error <= tol, and every row
    within its relative bound (see ROW_REL)."""
    err = bf16_err(got, ref) if tol == BF16_TOL else max_err(got, ref)
    rel = row_rel_violation(got, ref)
    say(f"  {label} max abs err {err:.3e}, worst row error / row bound {rel:.3f}")
    assert np.isfinite(np.asarray(got)).all()
    assert err <= tol, (label, err)
    assert rel <= 1.0, (label, rel)
    return err


def sample_rows(n, extra=(), seed=0, count=16):
    """Rows 0-7, tile edges, the middle, the last row, and seeded random rows."""
    rows = set(range(min(8, n)))
    for r in (31, 32, 63, 64, 127, 128, 255, 256, n // 2, n - 2, n - 1):
        if 0 <= r < n:
            rows.add(r)
    for r in extra:
        if 0 <= r < n:
            rows.add(int(r))
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.integers(0, n, size=count))
    return sorted(rows)


def sync():
    torch.cuda.synchronize()
