"""Pins for the quantisation oracle (oracle/quantize_ref.py), CPU only.

The oracle is checked against things other than itself: the e4m3fn closed
form (round trip of every code), ties and their neighbours, torch's CPU
float8 cast (an outside implementation), a hand-worked example, exact
rational arithmetic on small matrices, and invariants; planted mistakes are
rejected.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PT, RW = oracle.PER_TENSOR, oracle.ROWWISE


def to_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def test_encode_roundtrips_every_finite_code():
    assert np.array_equal(oracle.e4m3fn_encode_rne(oracle.decode(FINITE)), FINITE)


def test_ties_go_to_the_even_code_and_neighbours_to_the_nearest():
    v = oracle.decode(np.arange(0x7F, dtype=np.uint8))        # +0 .. 448, increasing
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2                                        # exact in fp64
    got = oracle.e4m3fn_encode_rne(mid)
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(got, want.astype(np.uint8))
    eps = (hi - lo) * 2.0 ** -10
    assert np.array_equal(oracle.e4m3fn_encode_rne(mid - eps), np.arange(0x7E, dtype=np.uint8))
    assert np.array_equal(oracle.e4m3fn_encode_rne(mid + eps), np.arange(1, 0x7F, dtype=np.uint8))
    assert np.array_equal(oracle.e4m3fn_encode_rne(-mid), want.astype(np.uint8) | 0x80)


def test_encode_matches_torch_cpu_cast():
    rng = np.random.default_rng(1)
    y = (rng.uniform(-448, 448, 300000) * np.exp2(rng.integers(-16, 1, 300000))).astype(np.float32)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode_rne(y.astype(np.float64)), want)


def _golden():
    x, rs, rc, ps, pc = [], None, [], None, []
    for line in open(os.path.join(GOLD, "quantize_handworked.txt")):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "x":
            x.append([float(t) for t in f[1:]])
        elif f[0] == "rowwise_scale_bits":
            rs = np.array([int(t, 16) for t in f[1:]], np.uint32)
        elif f[0] == "rowwise_codes":
            rc.append([int(t, 16) for t in f[1:]])
        elif f[0] == "per_tensor_scale_bits":
            ps = np.array([int(t, 16) for t in f[1:]], np.uint32)
        elif f[0] == "per_tensor_codes":
            pc.append([int(t, 16) for t in f[1:]])
    return np.array(x, np.float32), rs, np.array(rc, np.uint8), ps, np.array(pc, np.uint8)


def test_handworked_example():
    x, rs, rc, ps, pc = _golden()
    xb = to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_f64(xb), x.astype(np.float64))   # exact in bf16
    q, s = oracle.quantize_e4m3(xb, RW)
    assert np.array_equal(s.view(np.uint32), rs) and np.array_equal(q, rc)
    q, s = oracle.quantize_e4m3(xb, PT)
    assert np.array_equal(s.view(np.uint32), ps) and np.array_equal(q, pc)


# ---- exact rational brute force -------------------------------------------

def _rne_fp32(fr: Fraction) -> Fraction:
    """Nearest fp32 to a rational (ties to even), normal range and subnormals."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 23)                      # fp32 spacing at a
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * q


def _nearest_code(y: Fraction) -> int:
    """Brute force over every finite code: the nearest value, ties to the even code."""
    best = None
    for c in range(0x7F):
        d = abs(abs(y) - Fraction(oracle.e4m3fn_value(c)))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if y < 0 else 0)


def _brute(xb, mode):
    x = [[Fraction(float(v)) for v in row] for row in oracle.bf16_bits_to_f64(xb)]
    R = len(x)
    if mode == PT:
        amaxes = [max(abs(v) for row in x for v in row)] * R
    else:
        amaxes = [max(abs(v) for v in row) for row in x]
    scales = [_rne_fp32(a / 448) for a in amaxes]
    codes = np.zeros((R, len(x[0])), np.uint8)
    for i, row in enumerate(x):
        for j, v in enumerate(row):
            if scales[i] == 0:
                continue
            y = _rne_fp32(v / scales[i])
            y = max(min(y, Fraction(448)), Fraction(-448))
            c = _nearest_code(y)
            if y == 0 and float(v) == 0 and np.signbit(oracle.bf16_bits_to_f64(xb)[i, j]):
                c = 0x80
            codes[i, j] = c
    s = np.array([float(v) for v in (scales[:1] if mode == PT else scales)], np.float32)
    return codes, s


@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_exact_rationals(mode, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((4, 9)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (4, 1)))
    x[1, 3] = 0.0
    x[2, :] = 0.0                                       # an all-zero row
    x[3, 2] = -0.0
    xb = to_bf16_bits(x)
    q, s = oracle.quantize_e4m3(xb, mode)
    bq, bs = _brute(xb, mode)
    assert np.array_equal(s, bs)
    assert np.array_equal(q, bq)


# ---- invariants -------------------------------------------------------------

def _random_bits(rows, cols, seed):
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32) * 3.0)


def test_row_max_maps_to_448():
    xb = _random_bits(32, 257, 3)
    q, s = oracle.quantize_e4m3(xb, RW)
    x = oracle.bf16_bits_to_f64(xb)
    j = np.argmax(np.abs(x), axis=1)
    top = q[np.arange(32), j]
    assert np.all((top & 0x7F) == 0x7E)
    assert np.array_equal(top >> 7, (x[np.arange(32), j] < 0).astype(np.uint8))


def test_single_row_per_tensor_equals_rowwise():
    xb = _random_bits(1, 999, 4)
    a, sa = oracle.quantize_e4m3(xb, PT)
    b, sb = oracle.quantize_e4m3(xb, RW)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_power_of_two_invariance():
    xb = _random_bits(16, 300, 5)
    x = oracle.bf16_bits_to_f64(xb)
    xb4 = to_bf16_bits((x * 4.0).astype(np.float32))
    for mode in (PT, RW):
        q, s = oracle.quantize_e4m3(xb, mode)
        q4, s4 = oracle.quantize_e4m3(xb4, mode)
        assert np.array_equal(q, q4) and np.array_equal(s4, s * np.float32(4.0))


def test_dequantised_error_within_half_e4m3_spacing():
    xb = _random_bits(24, 512, 6)
    x = oracle.bf16_bits_to_f64(xb)
    q, s = oracle.quantize_e4m3(xb, RW)
    d = oracle.dequantize(q, s, RW)
    y = x / s.astype(np.float64)[:, None]
    a = np.abs(y)
    _, e = np.frexp(a)
    spacing = np.where(a >= 2.0 ** -6, np.ldexp(1.0, e - 4), 2.0 ** -9)
    # half an e4m3 spacing in y units, plus the fp32 rounding of y (relative 2^-24)
    bound = (0.5 * spacing + a * 2.0 ** -23) * s.astype(np.float64)[:, None]
    assert np.all(np.abs(d - x) <= bound)


def test_planted_mistakes_are_rejected():
    x, rs, rc, ps, pc = _golden()
    xb = to_bf16_bits(x)
    good, _ = oracle.quantize_e4m3(xb, RW)
    # truncation instead of ties-to-even
    trunc = oracle.e4m3fn_encode_rne(np.float64(1.0625) - 1e-12)
    assert trunc == 0x38 and oracle.e4m3fn_encode_rne(np.float64(1.1875)) == 0x3A
    # dividing by amax instead of amax / 448 would give codes that differ
    xf = oracle.bf16_bits_to_f64(xb)
    amax = np.max(np.abs(xf), axis=1)
    wrong = oracle.e4m3fn_encode_rne(np.clip(xf / amax[:, None], -448, 448))
    assert not np.array_equal(wrong, good)
    # multiplying by the fp32 reciprocal of the scale instead of dividing by it
    # differs from the correctly rounded division on some inputs
    rng = np.random.default_rng(7)
    xb2 = to_bf16_bits(rng.standard_normal((64, 512)).astype(np.float32))
    q, s = oracle.quantize_e4m3(xb2, RW)
    y_rcp = (oracle.bf16_bits_to_f64(xb2).astype(np.float32)
             * (np.float32(1.0) / s)[:, None]).astype(np.float64)
    q_rcp = oracle.e4m3fn_encode_rne(np.clip(y_rcp, -448, 448))
    assert not np.array_equal(q_rcp, q)
