"""The GPU parity tests bound the error of an attention output beyond the rounding of the
exact result to the output dtype (tests/_gpu.py, output_half_step and max_err). These CPU
tests pin that allowance: it is half the dtype's spacing (never less than the error of a
correct rounding, and reached exactly at ties) and nothing more."""
import numpy as np
import pytest
import torch

from tests._gpu import output_half_step


@pytest.mark.parametrize("dtype,p,emin", [(torch.bfloat16, 8, -126), (torch.float16, 11, -14)])
def test_half_step_is_the_rounding_error_bound(dtype, p, emin):
    rng = np.random.default_rng(5)
    # fp32 values across many binades (the kernels round from fp32), zero and powers of two
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-30, 12, 100000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, 1.0, 4.0, -4.0, 2.0 ** -14, 2.0 ** -24, 2.0 ** -130])]).astype(np.float64)
    rounded = torch.from_numpy(x.astype(np.float32)).to(dtype).double().numpy()
    hs = output_half_step(x, dtype)
    ok = np.isfinite(rounded)
    ratio = np.abs(rounded - x)[ok] / hs[ok]
    assert ratio.max() == 1.0   # a correct rounding never exceeds it, and ties reach it


def test_half_step_values():
    bf = output_half_step(np.array([4.2, -4.0, 3.99, 2.62, 1.0, 0.3, 0.0]), torch.bfloat16)
    np.testing.assert_array_equal(bf, [2.0 ** -6, 2.0 ** -6, 2.0 ** -7, 2.0 ** -7, 2.0 ** -8, 2.0 ** -10, 2.0 ** -134])
    hf = output_half_step(np.array([4.2, 1.0, 2.0 ** -20, 0.0]), torch.float16)
    np.testing.assert_array_equal(hf, [2.0 ** -9, 2.0 ** -11, 2.0 ** -25, 2.0 ** -25])


def test_no_bf16_value_lies_within_the_bare_bound_of_4_2():
    # The reason for the allowance: 4.2's bf16 neighbours are 4.1875 and 4.21875, both more
    # than 1e-2 away, so no bf16 output of an exact 4.2 meets a bare 1e-2 bound.
    lo, hi = 4.1875, 4.21875
    assert float(torch.tensor(lo, dtype=torch.bfloat16)) == lo and float(torch.tensor(hi, dtype=torch.bfloat16)) == hi
    assert float(torch.nextafter(torch.tensor(lo, dtype=torch.bfloat16), torch.tensor(5.0, dtype=torch.bfloat16))) == hi
    assert min(4.2 - lo, hi - 4.2) > 1e-2
    assert min(4.2 - lo, hi - 4.2) <= output_half_step(np.array([4.2]), torch.bfloat16)[0]
