"""Plain CPU oracle for dynamic FP8 (e4m3fn or e5m2) quantisation of a bf16 matrix.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

What it computes (the gist "matmul_fp8.py" (a-r-r-o-w), functions `get_scale`
and `benchmark`, which quantise the bf16 operands before the scaled multiply;
the producer step that pytorch PR #130422 "Inductor lowering for
`torch._scaled_mm`", Testing, says row-wise scaling lets the compiler fuse
with the preceding op):

  * amax = max |x| over the whole matrix (per-tensor) or over each row
    (row-wise: the gist's `amax(dim=1)` over a's K, and over K of b's N x K
    transpose); a bf16 value, hence exact in fp32.
  * scale = amax / quant_max in fp32 (`scale / quant_max`, quant_max =
    finfo(dtype).max: 448 for float8_e4m3fn, 57344 for float8_e5m2, the two
    dtypes the gist's quantisation branch accepts): one correctly rounded
    fp32 division.
  * y = x / scale in fp32 (the bf16 x is promoted to fp32 by the division
    with the fp32 scale): one correctly rounded fp32 division.
  * y is clamped to [-quant_max, quant_max] (`.clamp(quant_min, quant_max)`)
    and cast to the float8 format, round to nearest, ties to even.
  * Reading where the pages are silent: an all-zero row (or matrix) would
    give 0/0; it quantises to code 0x00 with scale 0 here (dequantises to
    the zero it came from).  Inputs are finite.

fp32 rounding of a quotient of two fp32 numbers: the fp64 quotient rounded
to fp32 is the correctly rounded fp32 quotient, because fp64 carries more
than 2*24 + 2 significant bits (double rounding is innocuous for division at
that width); both steps below use it and the tests check it against exact
rationals.
"""
from __future__ import annotations

import numpy as np

from .fp8_scaled_mm_ref import (E4M3FN, E5M2, PER_TENSOR, ROWWISE, bf16_bits_to_f64,
                                e4m3fn_value, e5m2_value)

E4M3_MAX = 448.0
E5M2_MAX = 57344.0


class _Format:
    """Rounding parameters of a float8 format: mantissa bits, smallest normal
    magnitude, subnormal spacing, largest finite value, the NaN code, and the
    values of the codes 0x00 .. max_code (+0 and every positive finite
    value), which the closed forms make strictly increasing: the index of a
    value is its code."""

    def __init__(self, name, mbits, min_normal, quantum, vmax, max_code, nan_code, value):
        self.name, self.mbits, self.min_normal, self.quantum = name, mbits, min_normal, quantum
        self.vmax, self.max_code, self.nan_code = vmax, max_code, nan_code
        self.pos_values = np.array([value(c) for c in range(max_code + 1)], dtype=np.float64)


FORMATS = {
    E4M3FN: _Format("e4m3fn", 3, 2.0 ** -6, 2.0 ** -9, E4M3_MAX, 0x7E, 0x7F, e4m3fn_value),
    E5M2: _Format("e5m2", 2, 2.0 ** -14, 2.0 ** -16, E5M2_MAX, 0x7B, 0x7E, e5m2_value),
}


def encode_rne(y: np.ndarray, fmt: int = E4M3FN) -> np.ndarray:
    """Round values (fp64 holding fp32 numbers, |y| <= the format's largest
    finite value, or NaN) to float8 codes with round to nearest, ties to even.

    Normal range |y| >= min_normal: with |y| in [2^e, 2^(e+1)) the spacing
    is 2^(e - mbits).  Below min_normal the spacing is the subnormal quantum.
    Dividing by a power of two is exact, np.rint rounds half to even, and a
    result equal to the next power of two is that binade's first value, which
    is also even.  Negative values (and -0) get the sign bit; NaN gives the
    format's positive NaN code (0x7F for e4m3fn, 0x7E for e5m2).
    """
    f = FORMATS[fmt]
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a[~np.isnan(a)] > f.vmax):
        raise ValueError(f"encode_rne expects |y| <= {f.vmax:g} for {f.name} (clamp first)")
    _, e = np.frexp(a)                         # a = m * 2^e, m in [0.5, 1)
    spacing = np.where(a >= f.min_normal, np.ldexp(1.0, e.astype(np.int64) - 1 - f.mbits),
                       f.quantum)
    with np.errstate(invalid="ignore"):
        r = np.rint(a / spacing) * spacing
    nan = np.isnan(r)
    r0 = np.where(nan, 0.0, r)
    idx = np.searchsorted(f.pos_values, r0)
    if not np.array_equal(f.pos_values[np.minimum(idx, f.max_code)], r0):
        raise AssertionError(f"rounded value is not an {f.name} value")
    codes = idx.astype(np.uint8)
    codes = np.where(np.signbit(y), codes | np.uint8(0x80), codes)
    codes = np.where(nan, np.uint8(f.nan_code), codes)
    return codes.astype(np.uint8)


def e4m3fn_encode_rne(y: np.ndarray) -> np.ndarray:
    """encode_rne for e4m3fn (|y| <= 448)."""
    return encode_rne(y, E4M3FN)


def _f32(x: np.ndarray) -> np.ndarray:
    """Round fp64 to the nearest fp32 (ties to even) and return it as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize(x_bits: np.ndarray, mode: int = ROWWISE, fmt: int = E4M3FN):
    """Quantise a rows x cols bf16 matrix (uint16 bit patterns) to `fmt`.

    Returns (codes uint8 [rows, cols], scale float32 [1] or [rows]), where
    scale = fp32(amax / quant_max) and codes = RNE(clamp(fp32(x / scale),
    -quant_max, quant_max)).  Follows the steps of the gist's `get_scale` /
    `benchmark`.
    """
    qmax = FORMATS[fmt].vmax
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("x must be rows x cols")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    if mode == PER_TENSOR:
        amax = np.array([np.max(np.abs(x))]) if x.size else np.zeros(1)
        s = _f32(amax / qmax)
        s_row = np.full(x.shape[0], s[0])
    elif mode == ROWWISE:
        amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
        s = _f32(amax / qmax)
        s_row = s
    else:
        raise ValueError(f"unknown scaling mode {mode}")
    with np.errstate(invalid="ignore", divide="ignore"):
        y = _f32(x / s_row[:, None])
    y = np.where(s_row[:, None] == 0.0, 0.0, y)      # all-zero rows: 0 / 0 -> code 0
    y = np.clip(y, -qmax, qmax)
    return encode_rne(y, fmt), s.astype(np.float32)


def quantize_e4m3(x_bits: np.ndarray, mode: int = ROWWISE):
    """quantize() to e4m3fn (quant_max 448)."""
    return quantize(x_bits, mode, E4M3FN)


def dequantize(codes: np.ndarray, scale: np.ndarray, mode: int = ROWWISE,
               fmt: int = E4M3FN) -> np.ndarray:
    """fp64 value of codes * scale (row scales broadcast over columns)."""
    from .fp8_scaled_mm_ref import decode
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    d = decode(codes, fmt)
    return d * (s[0] if mode == PER_TENSOR else s[:, None])
