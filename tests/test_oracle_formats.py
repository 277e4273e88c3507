"""Pins of the oracle's storage formats: closed forms, exhaustive brute force, library casts."""
import numpy as np
import pytest
import torch

from oracle import formats

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_e4m3_closed_form_values():
    d = formats.e4m3_to_f64
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x38) == 1.0                  # exponent field 7 = bias
    assert d(0x7E) == 448.0                # largest finite
    assert d(0xFE) == -448.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert np.isfinite(d(np.arange(256)[(np.arange(256) & 0x7F) != 0x7F])).all()


def test_e4m3_decode_matches_torch_float8_e4m3fn_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_to_f64(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == lib) | (np.isnan(ours) & np.isnan(lib))
    assert same.all()


def test_e4m3_positive_codes_are_increasing():
    v = formats.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert (np.diff(v) > 0).all()


def _brute_force_encode(x):
    """Nearest finite E4M3FN value by exhaustive search; ties to the even code; saturating."""
    codes = np.arange(0x7F)
    vals = formats.e4m3_to_f64(codes.astype(np.uint8))
    out = np.empty(len(x), dtype=np.uint8)
    for i, xi in enumerate(x):
        if np.isnan(xi):
            out[i] = 0x7F | (0x80 if np.signbit(xi) else 0)
            continue
        a = min(abs(xi), 448.0)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | (0x80 if np.signbit(xi) else 0)
    return out


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_e4m3_encode_matches_brute_force_on_every_16bit_pattern(fmt):
    x = formats.to_f64(ALL16, fmt)
    ours = formats.e4m3_encode(x)
    # Brute force on a strided subset plus every value near the format's interesting range.
    near = np.flatnonzero(np.abs(np.nan_to_num(x, nan=0.0, posinf=1e9, neginf=-1e9)) <= 600.0)
    pick = np.union1d(np.arange(0, 1 << 16, 7), near[::3])
    np.testing.assert_array_equal(ours[pick], _brute_force_encode(x[pick]))


def test_e4m3_encode_matches_torch_cast_inside_the_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([formats.to_f64(ALL16, "bf16"), formats.to_f64(ALL16, "f16"),
                        rng.standard_normal(20000).astype(np.float32) * 50])
    x = x[np.isfinite(x) & (np.abs(x) <= 448.0)]
    ours = formats.e4m3_encode(x)
    lib = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, lib)


def test_e4m3_encode_saturates_and_keeps_nan_and_zero_signs():
    enc = formats.e4m3_encode
    assert enc(448.0) == 0x7E and enc(449.0) == 0x7E and enc(1e30) == 0x7E and enc(np.inf) == 0x7E
    assert enc(-464.0) == 0xFE and enc(-np.inf) == 0xFE
    assert enc(np.nan) == 0x7F and enc(-np.nan) == 0xFF
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -11) == 0x00         # below half the smallest subnormal
    assert enc(2.0 ** -10) == 0x00         # exact tie between 0 and 2^-9 -> even code 0
    assert enc(3 * 2.0 ** -10) == 0x02     # tie between codes 1 and 2 -> even code 2
    assert enc(1.0625) == 0x38             # tie between 1.0 and 1.125 -> even mantissa
    assert enc(1.1875) == 0x3A             # tie between 1.125 and 1.25 -> even mantissa


def test_quotient_rounding_equals_ieee_fp32_division():
    # fl32(x / s) computed in float64 then rounded equals the IEEE binary32 quotient.
    x = formats.to_f64(ALL16, "bf16")
    x = x[np.isfinite(x)]
    for s in (np.float32(1 / 128), np.float32(0.0134), np.float32(3.7)):
        ours = formats.round_to_f32(x / float(s))
        with np.errstate(over="ignore", under="ignore"):
            ieee = (x.astype(np.float32) / s).astype(np.float64)
        np.testing.assert_array_equal(ours, ieee)


def test_bf16_and_f16_decoders():
    assert formats.bf16_to_f64(0x3F80) == 1.0
    assert formats.bf16_to_f64(0xC000) == -2.0
    assert formats.bf16_to_f64(0x0001) == 2.0 ** -133
    assert formats.f16_to_f64(0x3C00) == 1.0
    assert formats.f16_to_f64(0x7BFF) == 65504.0
    assert formats.f16_to_f64(0x0001) == 2.0 ** -24
    lib = torch.from_numpy(ALL16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = formats.bf16_to_f64(ALL16)
    assert ((ours == lib) | (np.isnan(ours) & np.isnan(lib))).all()
