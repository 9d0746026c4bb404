"""Plain CPU oracle for the FP8 (e4m3fn, e5m2) scaled matrix multiply.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it.

What it computes (the plain definition of the method):

    out[m, n] = RNE_bf16( s[m, n] * sum_k dec(A[m, k]) * dec(B[n, k])  (+ bias[n]) )

  * A is M x K and B is N x K, float8 codes with K fastest: e4m3fn, or
    e5m2 (the gist's `benchmark` takes either dtype), each operand its own.  B is the
    K x N column-major right operand of the pages ("TN"): the gist
    "matmul_fp8.py", function `benchmark`, makes b column-major before the
    call, and the row-wise kernel PR (pytorch #125204, Summary) supports only
    TN and scales B along its fast dimension.
  * s[m, n] = scale_a * scale_b (per-tensor, gist `matmul_fp8_kernel`, the
    scalar scale branch) or scale_a[m] * scale_b[n] (row-wise, same kernel's
    per-row branch; PR #125204 Summary: scale of x has length M, scale of y
    length N).
  * The products are accumulated in fp32 on the GPU (gist: the accumulator is
    float32 and every `tl.dot` asks for float32 output); here they are
    accumulated in fp64, which is exact (see `scaled_mm`).
  * The scale multiplies the accumulated sum once, after the K loop, and the
    result is cast to the output dtype (gist `matmul_fp8_kernel`, after the K
    loop).  The bias is added after scaling, unscaled (PR #142045 Summary: the
    plan is to apply scaling and bias as epilogues; reading: bias is not
    multiplied by the scale).
  * The bf16 cast is round-to-nearest-even, done once, directly from fp64.

Every piece is pinned by tests against closed forms, brute force with exact
rationals, invariants and torch's CPU casts (as an outside library).
"""
from __future__ import annotations

import numpy as np

PER_TENSOR = 0
ROWWISE = 1

# Operand formats.  The gist's `benchmark` accepts float8_e4m3fn or
# float8_e5m2 as the operand dtype (its quantisation branch lists both);
# A and B may also differ.
E4M3FN = 0
E5M2 = 1
FORMAT_NAMES = {E4M3FN: "e4m3fn", E5M2: "e5m2"}


def e4m3fn_value(code: int) -> float:
    """Closed-form value of one OCP float8 e4m3fn byte.

    Bit layout s eeee mmm, exponent bias 7.  Exponent field 15 with mantissa
    7 is NaN (there is no infinity); exponent field 0 is subnormal,
    m * 2^-9; otherwise (1 + m/8) * 2^(e-7).  The largest finite magnitude is
    448 (the gist quantises to torch.finfo(float8_e4m3fn).max, which is 448).
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e5m2_value(code: int) -> float:
    """Closed-form value of one OCP float8 e5m2 byte.

    Bit layout s eeeee mm, exponent bias 15, IEEE-style specials: exponent
    field 31 is infinity (mantissa 0) or NaN (mantissa 1..3); exponent field
    0 is subnormal, m * 2^-16; otherwise (1 + m/4) * 2^(e-15).  The largest
    finite magnitude is 1.75 * 2^15 = 57344 (torch.finfo(float8_e5m2).max,
    the clamp limit of the gist's quantisation for that dtype).
    """
    s = (code >> 7) & 1
    e = (code >> 2) & 0x1F
    m = code & 0x3
    sign = -1.0 if s else 1.0
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * m * 2.0 ** -16
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


def e4m3fn_decode_table() -> np.ndarray:
    """fp64 value of every byte code 0..255."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def e5m2_decode_table() -> np.ndarray:
    """fp64 value of every e5m2 byte code 0..255."""
    return np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)


_DECODE = e4m3fn_decode_table()
_DECODE_E5M2 = e5m2_decode_table()

# Every finite value of a format is an integer multiple of 2^-UNIT_EXP: its
# smallest subnormal.
UNIT_EXP = {E4M3FN: 9, E5M2: 16}


def decode(codes: np.ndarray, fmt: int = E4M3FN) -> np.ndarray:
    if fmt == E4M3FN:
        table = _DECODE
    elif fmt == E5M2:
        table = _DECODE_E5M2
    else:
        raise ValueError(f"unknown operand format {fmt}")
    return table[np.asarray(codes, dtype=np.uint8)]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """A bf16 pattern is the top half of the fp32 pattern with the same value."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_rne(y: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, exponent range of fp32)
    with round-to-nearest, ties-to-even, in one step; return bit patterns.

    For |y| in [2^e, 2^(e+1)) the bf16 spacing is 2^(e-7); below the smallest
    normal 2^-126 the spacing stays 2^-133 (subnormals).  Dividing by the
    spacing is exact (a power of two), np.rint rounds half to even, and the
    multiply back is exact.  A result of 2^128 or more is an overflow to
    infinity (that is where RNE sends values from (2 - 2^-8) * 2^127 up).
    NaN becomes the quiet NaN 0x7FC0.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, e = np.frexp(a)                     # a = f * 2^e with f in [0.5, 1)
    exp = np.maximum(e.astype(np.int64) - 1, -126)
    spacing = np.ldexp(1.0, exp - 7)
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(a / spacing) * spacing
        r32 = r.astype(np.float32)          # exact below 2^128, inf at 2^128
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(np.signbit(y), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(y), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def _exact_integer_acc(da: np.ndarray, db: np.ndarray, qa: int, qb: int) -> np.ndarray:
    """sum_k da[m, k] * db[n, k] for finite values that are integer multiples
    of 2^-qa and 2^-qb, formed exactly in integers and rounded once to fp64.

    With na = da * 2^qa and nb = db * 2^qb (integers, |na|, |nb| < 2^32 for
    both formats), nb is split as hi * 2^16 + lo with 0 <= lo < 2^16 and
    |hi| < 2^16.  Each of sum_k na*hi and sum_k na*lo then stays below
    2^32 * 2^16 * K <= 2^63 for K <= 32768, so both int64 products are exact;
    they are joined as Python integers and converted to fp64 once (Python's
    int -> float conversion rounds to nearest even), then scaled by the exact
    power of two 2^-(qa + qb).
    """
    na = np.rint(np.ldexp(da, qa)).astype(np.int64)
    nb = np.rint(np.ldexp(db, qb)).astype(np.int64)
    hi = nb >> 16                         # floor division by 2^16
    lo = nb & 0xFFFF
    s_hi = na @ hi.T
    s_lo = na @ lo.T
    total = s_hi.astype(object) * 65536 + s_lo.astype(object)
    acc = np.array([float(v) for v in total.ravel()], dtype=np.float64).reshape(total.shape)
    return np.ldexp(acc, -(qa + qb))


def scaled_mm(a, b, scale_a, scale_b, bias=None, mode=PER_TENSOR, rows=None, cols=None,
              a_format=E4M3FN, b_format=E4M3FN):
    """Reference result for out[rows][:, cols] (all rows/cols by default).

    a: uint8 [M, K] codes; b: uint8 [N, K] codes; scale_a/scale_b: float32
    arrays of length 1 (per-tensor) or M / N (row-wise); bias: uint16 [N] bf16
    bits or None; a_format / b_format: E4M3FN (default) or E5M2.

    Returns a dict with
      bits : uint16 [m, n]  the bf16 output
      y    : float64 [m, n] the value before the bf16 rounding
      acc  : float64 [m, n] sum_k dec(a) dec(b)          (exact)
      mag  : float64 [m, n] sum_k |dec(a)| |dec(b)|      (exact)
      s    : float64 [m, n] the scale applied to acc

    Exactness of acc: every finite e4m3fn value is an integer multiple of
    2^-9 with magnitude at most 448 = 229376 * 2^-9, so each product is an
    integer multiple of 2^-18 below 2^36 units, and any partial sum over
    K <= 2^16 terms stays below 2^52 units.  All of them are fp64 numbers, so
    the fp64 sum is exact in any order; the matrix product below is just a
    convenient way to form it.

    With an e5m2 operand that argument fails (e5m2 spans 2^-16 .. 57344, so a
    sum can need more than 53 bits); acc is then the exact integer sum of
    `_exact_integer_acc` rounded once to fp64 (relative error <= 2^-53), for
    K <= 32768, and mag is the fp64 matrix product of the magnitudes (a
    tolerance term, relative error below K * 2^-53).  Non-finite codes are
    taken out of both sums and decide acc by the IEEE 754 rules below.
    """
    a = np.asarray(a, dtype=np.uint8)
    b = np.asarray(b, dtype=np.uint8)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("a must be M x K and b N x K")
    M, K = a.shape
    N = b.shape[0]
    if K > 65536:
        raise ValueError("exact fp64 accumulation is only argued for K <= 65536")
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N) if cols is None else np.asarray(cols, dtype=np.int64)

    da = decode(a[rows], a_format)           # [m, K]
    db = decode(b[cols], b_format)           # [n, K]
    # Non-finite codes (NaN in both formats: e4m3fn 0x7F / 0xFF, e5m2
    # 0x7D..0x7F / 0xFD..0xFF; +-infinity in e5m2 only: 0x7C / 0xFC) follow
    # IEEE 754 arithmetic, written out here rather than left to the
    # matrix-product library:
    #   a product is NaN if a factor is NaN, or one factor is infinite and the
    #   other zero; it is infinite, with the sign of the factors' signs'
    #   product, if a factor is infinite and the other non-zero;
    #   a sum is NaN if a term is NaN or it has both a +inf and a -inf term,
    #   else +-inf if it has an infinite term, else the finite sum.
    # Which of these holds for (m, n) is an "any over k" of elementwise
    # conditions on row m of A and row n of B; the finite sums are formed over
    # the other values, with every non-finite value replaced by 0.
    fa, fb = np.isfinite(da), np.isfinite(db)
    special = not (fa.all() and fb.all())
    if special:
        def any_k(x, y):   # [m, n]: some k with x[m, k] and y[n, k]
            return (x.astype(np.int64) @ y.astype(np.int64).T) > 0
        nan_a, nan_b = np.isnan(da), np.isnan(db)
        inf_a, inf_b = np.isinf(da), np.isinf(db)
        zero_a, zero_b = da == 0, db == 0
        pos_a, pos_b = ~nan_a & (da > 0), ~nan_b & (db > 0)
        neg_a, neg_b = ~nan_a & (da < 0), ~nan_b & (db < 0)
        nan_mask = (nan_a.any(axis=1)[:, None] | nan_b.any(axis=1)[None, :]
                    | any_k(inf_a, zero_b) | any_k(zero_a, inf_b))
        pinf = (any_k(inf_a & pos_a, pos_b) | any_k(inf_a & neg_a, neg_b)
                | any_k(pos_a, inf_b & pos_b) | any_k(neg_a, inf_b & neg_b))
        ninf = (any_k(inf_a & pos_a, neg_b) | any_k(inf_a & neg_a, pos_b)
                | any_k(pos_a, inf_b & neg_b) | any_k(neg_a, inf_b & pos_b))
        nan_mask |= pinf & ninf
        da = np.where(fa, da, 0.0)
        db = np.where(fb, db, 0.0)
    if a_format == E4M3FN and b_format == E4M3FN:
        acc = da @ db.T
    else:
        if K > 32768:
            raise ValueError("the integer accumulation is only argued for K <= 32768")
        acc = _exact_integer_acc(da, db, UNIT_EXP[a_format], UNIT_EXP[b_format])
    mag = np.abs(da) @ np.abs(db).T
    if special:
        acc = np.where(pinf, np.inf, acc)
        acc = np.where(ninf, -np.inf, acc)
        acc = np.where(nan_mask, np.nan, acc)

    sa = np.asarray(scale_a, dtype=np.float32).astype(np.float64).reshape(-1)
    sb = np.asarray(scale_b, dtype=np.float32).astype(np.float64).reshape(-1)
    if mode == PER_TENSOR:
        if sa.size != 1 or sb.size != 1:
            raise ValueError("per-tensor scales must have one element each")
        s = np.full(acc.shape, sa[0] * sb[0])
    elif mode == ROWWISE:
        if sa.size != M or sb.size != N:
            raise ValueError("row-wise scales must have M and N elements")
        # The product of two fp32 numbers is exact in fp64.
        s = sa[rows][:, None] * sb[cols][None, :]
    else:
        raise ValueError(f"unknown scaling mode {mode}")

    with np.errstate(invalid="ignore"):      # 0 * inf and inf - inf are NaN, as IEEE 754 has them
        y = s * acc
        if bias is not None:
            y = y + bf16_bits_to_f64(np.asarray(bias, dtype=np.uint16)[cols])[None, :]
    return {"bits": f64_to_bf16_rne(y), "y": y, "acc": acc, "mag": mag, "s": s}
