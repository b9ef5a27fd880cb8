"""The per-row parity bar used for sampled rows deep into long sequences
rejects the failures the absolute 1e-2 bound alone would accept there: a
zeroed row, a row scaled by a few percent, a row from the wrong position.
(CPU only: it exercises the checker on synthetic late-row magnitudes.)"""

import numpy as np
import pytest

from tests.gpu_util import BF16_TOL, ROW_ABS, ROW_REL, check_rows, max_err, row_rel_violation


def _late_rows(seed=0, rows=6, d=128, scale=1.5e-3):
    # outputs of late rows of a long causal head with N(0,1) values: ~1/sqrt(n)
    return np.random.default_rng(seed).standard_normal((rows, d)) * scale


def test_bf16_rounding_of_a_late_row_passes():
    ref = _late_rows()
    import torch
    got = torch.tensor(ref, dtype=torch.float32).to(torch.bfloat16).float().numpy()
    check_rows(got, ref)


@pytest.mark.parametrize("mistake", ["zero", "scale", "other_row"])
def test_late_row_mistakes_fail(mistake):
    ref = _late_rows()
    if mistake == "zero":
        got = np.zeros_like(ref)
    elif mistake == "scale":
        got = ref * 1.05
    else:
        got = _late_rows(seed=1)
    assert max_err(got, ref) <= BF16_TOL        # the absolute bound alone accepts it
    assert row_rel_violation(got, ref) > 1.0
    with pytest.raises(AssertionError):
        check_rows(got, ref)


def test_bound_constants():
    assert ROW_REL == 2.0 ** -6 and ROW_ABS == 1e-4
