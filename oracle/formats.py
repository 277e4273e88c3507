"""Storage formats of the KV cache, written out from their definitions.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.

The pages say the cache is held in FP16/BF16 and, on newer GPUs, in FP8, which
halves KV memory ("vLLM推理引擎PagedAttention原理与性能优化实战", §5.2, and
"vLLM 是什么…", §五 误解二). They do not fix the FP8 flavour; this oracle takes
OCP E4M3FN (bias 7, no infinities, NaN = S.1111.111, largest finite 448,
smallest subnormal 2^-9), with a per-tensor fp32 scale: stored code =
encode(fl32(x / scale)) rounded to nearest, ties to the even code, saturating at
+-448; the value read back is decode(code) * scale.

All decoders return float64 arrays, which hold every value of these formats
exactly.
"""
from __future__ import annotations

import numpy as np

F16 = "f16"
BF16 = "bf16"
FP8_E4M3 = "fp8_e4m3"
FORMATS = (F16, BF16, FP8_E4M3)

# Raw storage type of each format (the kernels see the bits, never a numpy float).
STORAGE = {F16: np.uint16, BF16: np.uint16, FP8_E4M3: np.uint8}

E4M3_MAX = 448.0


def f16_to_f64(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> exact float64 values.

    A bfloat16 is, by definition, the upper half of an IEEE binary32 word.
    """
    wide = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes) -> np.ndarray:
    """OCP E4M3FN codes -> exact float64 values (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = (1.0 + mant / 8.0) * np.exp2(exp_field.astype(np.float64) - 7.0)
    subnormal = mant * 2.0 ** -9
    mag = np.where(exp_field == 0, subnormal, normal)
    mag = np.where((exp_field == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def _e4m3_positive_table():
    """Codes 0x00..0x7E (every non-negative finite E4M3FN value), ascending."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return codes, e4m3_to_f64(codes)


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values (each an exact fp32 value) to OCP E4M3FN codes.

    Nearest finite code; a tie goes to the even code (the even mantissa);
    magnitudes past the largest finite value saturate to +-448 (infinities too);
    NaN maps to the NaN code with the input's sign bit. The sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    codes, values = _e4m3_positive_table()
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.searchsorted(values, a, side="left")           # first value >= a
    hi = np.minimum(hi, len(values) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - values[lo]
    d_hi = values[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0))
    mag_code = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    mag_code = np.where(nan, np.uint8(0x7F), mag_code)
    return (mag_code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def to_f64(bits, fmt: str) -> np.ndarray:
    if fmt == F16:
        return f16_to_f64(bits)
    if fmt == BF16:
        return bf16_to_f64(bits)
    if fmt == FP8_E4M3:
        return e4m3_to_f64(bits)
    raise ValueError(f"unknown format {fmt!r}")


def round_to_f32(x) -> np.ndarray:
    """Round float64 values to the nearest binary32 (ties to even), as float64."""
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
