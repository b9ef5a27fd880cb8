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
    err = max_err(got, ref)
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
