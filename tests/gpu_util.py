"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import sys

import numpy as np
import torch

BF16_TOL = 1e-2     # max abs error for bf16 inputs (fp32 accumulation)
F32_TOL = 1e-4      # max abs error for fp32 inputs


def to_np(t):
    """Exact float32 copy of a (bf16 or fp32) tensor as numpy."""
    return t.detach().float().cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_err(got, ref):
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)))


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
