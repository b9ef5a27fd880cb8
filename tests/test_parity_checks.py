"""The per-row parity bar used for sampled rows deep into long sequences
rejects the failures the absolute 1e-2 bound alone would accept there: a
zeroed row, a row scaled by a few percent, a row from the wrong position.
(CPU only: it exercises the checker on synthetic late-row magnitudes.)"""

import numpy as np
import pytest

from tests.gpu_util import (BF16_TOL, ROW_ABS, ROW_REL, bf16_err, bf16_half_ulp, check_rows, max_err,
                            row_rel_violation)


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


# The bf16 reading of the 1e-2 bound (tests/gpu_util.py): an output is a bf16
# value, and at |x| >= 4 the bf16 values are 2^-5 apart, so the correctly
# rounded exact result itself can be up to 1.56e-2 away.

def _bf16(x):
    import torch
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_no_bf16_value_meets_the_plain_bound_past_four():
    # an exact output value of a GPU parity case (bf16 prefill, d = 128, 127
    # rows, row 2): both neighbouring bf16 values are more than 1e-2 away
    ref = np.array([-4.04279])
    lo, hi = -4.0625, -4.03125
    assert lo < ref[0] < hi and hi - lo == 2.0 ** -5
    assert min(abs(ref[0] - lo), abs(ref[0] - hi)) > BF16_TOL
    assert _bf16(ref)[0] == hi                                  # correctly rounded
    assert bf16_err(_bf16(ref), ref) <= BF16_TOL                # accepted by the reading
    assert bf16_err(np.array([lo]), ref) > BF16_TOL             # the other neighbour is not


def test_bf16_reading_is_the_plain_bound_below_four():
    rng = np.random.default_rng(3)
    ref = rng.uniform(-3.999, 3.999, size=4000)
    got = ref + rng.uniform(-2e-2, 2e-2, size=ref.shape)
    for i in range(0, 4000, 50):
        assert bf16_err(got[i:i + 50], ref[i:i + 50]) == max_err(got[i:i + 50], ref[i:i + 50])


def test_correctly_rounded_outputs_pass_at_every_magnitude():
    rng = np.random.default_rng(4)
    ref = rng.uniform(-64, 64, size=20000)
    assert bf16_err(_bf16(ref), ref) <= BF16_TOL
    # an output one bf16 ulp further from the exact value than the correctly
    # rounded one fails wherever that ulp exceeds the bound (|x| >= 2)
    big = ref[np.abs(ref) >= 2.0]
    rounded = _bf16(big)
    away = np.where(rounded >= big, 1.0, -1.0)
    off = rounded + away * 2.0 * bf16_half_ulp(big)
    for i in range(0, big.size, 200):
        assert bf16_err(off[i:i + 200], big[i:i + 200]) > BF16_TOL
