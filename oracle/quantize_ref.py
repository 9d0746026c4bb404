"""Plain CPU oracle for dynamic FP8 (e4m3fn) quantisation of a bf16 matrix.

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
  * scale = amax / 448 in fp32 (`scale / quant_max`, quant_max =
    finfo(float8_e4m3fn).max = 448): one correctly rounded fp32 division.
  * y = x / scale in fp32 (the bf16 x is promoted to fp32 by the division
    with the fp32 scale): one correctly rounded fp32 division.
  * y is clamped to [-448, 448] (`.clamp(quant_min, quant_max)`) and cast to
    e4m3fn, round to nearest, ties to even.
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

from .fp8_scaled_mm_ref import PER_TENSOR, ROWWISE, bf16_bits_to_f64, e4m3fn_value

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6      # smallest normal e4m3fn magnitude (exponent field 1)
_SUB_QUANTUM = 2.0 ** -9     # spacing of the subnormals


# Values of the codes 0x00 .. 0x7E (+0 and every positive finite value), which
# the closed form makes strictly increasing: the index of a value is its code.
_POS_VALUES = np.array([e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)


def e4m3fn_encode_rne(y: np.ndarray) -> np.ndarray:
    """Round values (fp64 holding fp32 numbers, |y| <= 448 or NaN) to e4m3fn
    codes with round to nearest, ties to even.

    Normal range |y| >= 2^-6: with |y| in [2^e, 2^(e+1)) the spacing is
    2^(e-3) (3 mantissa bits).  Below 2^-6 the spacing is the subnormal
    quantum 2^-9.  Dividing by a power of two is exact, np.rint rounds half
    to even, and a result equal to the next power of two is that binade's
    first value, which is also even.  Negative values (and -0) get the sign
    bit; NaN gives 0x7F.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a[~np.isnan(a)] > E4M3_MAX):
        raise ValueError("e4m3fn_encode_rne expects |y| <= 448 (clamp first)")
    _, e = np.frexp(a)                         # a = f * 2^e, f in [0.5, 1)
    spacing = np.where(a >= _MIN_NORMAL, np.ldexp(1.0, e.astype(np.int64) - 1 - 3), _SUB_QUANTUM)
    with np.errstate(invalid="ignore"):
        r = np.rint(a / spacing) * spacing
    nan = np.isnan(r)
    r0 = np.where(nan, 0.0, r)
    idx = np.searchsorted(_POS_VALUES, r0)
    if not np.array_equal(_POS_VALUES[np.minimum(idx, 0x7E)], r0):
        raise AssertionError("rounded value is not an e4m3fn value")
    codes = idx.astype(np.uint8)
    codes = np.where(np.signbit(y), codes | np.uint8(0x80), codes)
    codes = np.where(nan, np.uint8(0x7F), codes)
    return codes.astype(np.uint8)


def _f32(x: np.ndarray) -> np.ndarray:
    """Round fp64 to the nearest fp32 (ties to even) and return it as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize_e4m3(x_bits: np.ndarray, mode: int = ROWWISE):
    """Quantise a rows x cols bf16 matrix (uint16 bit patterns).

    Returns (codes uint8 [rows, cols], scale float32 [1] or [rows]), where
    scale = fp32(amax / 448) and codes = e4m3fn_RNE(clamp(fp32(x / scale),
    -448, 448)).  Follows the steps of the gist's `get_scale` / `benchmark`.
    """
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("x must be rows x cols")
    if not np.all(np.isfinite(x)):
        raise ValueError("inputs must be finite")
    if mode == PER_TENSOR:
        amax = np.array([np.max(np.abs(x))]) if x.size else np.zeros(1)
        s = _f32(amax / E4M3_MAX)
        s_row = np.full(x.shape[0], s[0])
    elif mode == ROWWISE:
        amax = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0])
        s = _f32(amax / E4M3_MAX)
        s_row = s
    else:
        raise ValueError(f"unknown scaling mode {mode}")
    with np.errstate(invalid="ignore", divide="ignore"):
        y = _f32(x / s_row[:, None])
    y = np.where(s_row[:, None] == 0.0, 0.0, y)      # all-zero rows: 0 / 0 -> code 0
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    return e4m3fn_encode_rne(y), s.astype(np.float32)


def dequantize(codes: np.ndarray, scale: np.ndarray, mode: int = ROWWISE) -> np.ndarray:
    """fp64 value of codes * scale (row scales broadcast over columns)."""
    from .fp8_scaled_mm_ref import decode
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    d = decode(codes)
    return d * (s[0] if mode == PER_TENSOR else s[:, None])
