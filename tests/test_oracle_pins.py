"""Pins for the CPU oracle: closed forms, published special values, exact
rational brute force, invariants, and torch's CPU casts as an outside library.

None of these tests touches the GPU path.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_scaled_mm_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PT, RW = oracle.PER_TENSOR, oracle.ROWWISE


# ---------------------------------------------------------------- decode ---

def _golden_codes():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3fn_special_codes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, val = line.split()
            rows.append((int(code, 16), val))
    return rows


def test_decode_golden_special_codes():
    rows = _golden_codes()
    assert len(rows) >= 15
    for code, val in rows:
        got = oracle.e4m3fn_value(code)
        if val == "nan":
            assert math.isnan(got), hex(code)
            continue
        want = Fraction(val)
        assert Fraction(got) == want, (hex(code), got, want)
        if val.startswith("-0"):
            assert math.copysign(1.0, got) < 0


def test_decode_class_counts():
    t = oracle.e4m3fn_decode_table()
    nan = np.isnan(t)
    zero = t == 0
    finite = t[~nan]
    sub = (np.abs(finite) > 0) & (np.abs(finite) < 2.0 ** -6)
    assert nan.sum() == 2 and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert zero.sum() == 2
    assert sub.sum() == 14
    assert (np.abs(finite) >= 2.0 ** -6).sum() == 238
    assert np.nanmax(t) == 448.0 and np.nanmin(t) == -448.0


def test_decode_monotone_symmetric_continuous():
    t = oracle.e4m3fn_decode_table()
    pos = t[0x00:0x7F]
    assert np.all(np.diff(pos) > 0)
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert t[c ^ 0x80] == -t[c]
    # the last subnormal plus one quantum is the first normal
    assert t[0x07] + 2.0 ** -9 == t[0x08]
    # within a binade the step is 1/8 of the binade's lower end
    for e in range(1, 15):
        lo = 2.0 ** (e - 7)
        for m in range(8):
            c = (e << 3) | m
            assert t[c] == lo * (1 + m / 8)


def test_decode_matches_torch_cpu_cast():
    """torch's float8_e4m3fn is an independent implementation of OCP e4m3fn."""
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.e4m3fn_decode_table()
    assert np.array_equal(np.isnan(tv), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(tv[ok], t[ok])
    assert np.array_equal(np.signbit(tv[ok]), np.signbit(t[ok]))


# ---------------------------------------------------------- bf16 rounding ---

def _rne_fraction(x: Fraction) -> int:
    """bf16 bits of x by the textbook definition, on exact rationals: pick the
    nearer of the two bf16 neighbours, the one with an even last bit on a tie,
    and overflow to infinity past the midpoint above the largest finite."""
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    if a == 0:
        return sign
    # find e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    n = a / q
    lo = n.numerator // n.denominator
    frac = n - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    v = lo * q
    top = (2 - Fraction(1, 2 ** 7)) * Fraction(2) ** 127
    if v > top:
        return sign | 0x7F80
    # assemble bits from the integer significand
    if e == -126 and lo < 128:
        return sign | lo                         # subnormal (or zero)
    if lo == 256:
        lo, e = 128, e + 1
    if e > 127:
        return sign | 0x7F80
    return sign | ((e + 127) << 7) | (lo - 128)


def _golden_rne():
    rows = []
    with open(os.path.join(GOLDEN, "bf16_rne_cases.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            expr, bits = line.rsplit(None, 1)
            rows.append((expr.strip(), int(bits, 16)))
    return rows


def test_bf16_rne_golden_cases():
    rows = _golden_rne()
    assert len(rows) >= 15
    for expr, bits in rows:
        exact = eval(expr.replace("2**", "Fraction(2)**"), {"Fraction": Fraction})
        exact = Fraction(exact)
        if expr != "-0.0":                         # a Fraction has no signed zero
            assert _rne_fraction(exact) == bits, expr
        x = float(exact) if expr != "-0.0" else -0.0
        assert Fraction(x) == exact, expr          # the inputs are fp64-exact
        got = int(oracle.f64_to_bf16_rne(np.array([x]))[0])
        assert got == bits, (expr, hex(got), hex(bits))


def test_bf16_rne_matches_torch_on_fp32_inputs():
    """For fp32 inputs, direct fp64->bf16 RNE must equal torch's fp32->bf16
    cast.  Inputs sweep every exponent, random mantissas, and exact ties."""
    rng = np.random.Generator(np.random.PCG64(7))
    n = 1 << 20
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    ties = bits.copy()
    ties[: n // 2] = (ties[: n // 2] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    allbits = np.concatenate([bits, ties])
    f = allbits.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16_rne(f.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(f[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_bf16_rne_matches_exact_rationals_on_fp64_inputs():
    rng = np.random.Generator(np.random.PCG64(11))
    xs = []
    for _ in range(4000):
        e = int(rng.integers(-140, 128))
        m = float(rng.random()) + 1.0
        x = math.ldexp(m, e) * (1 if rng.random() < 0.5 else -1)
        xs.append(x)
    # fp64 values within a few ulps of bf16 ties, where rounding via fp32 would fail
    for _ in range(2000):
        e = int(rng.integers(-120, 120))
        mant = int(rng.integers(128, 256))
        tie = math.ldexp(mant + 0.5, e - 7)
        xs.append(math.nextafter(tie, math.inf))
        xs.append(math.nextafter(tie, -math.inf))
        xs.append(tie)
    got = oracle.f64_to_bf16_rne(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == _rne_fraction(Fraction(x)), x


def test_bf16_nan_and_overflow():
    got = oracle.f64_to_bf16_rne(np.array([np.nan, np.inf, -np.inf, 1e300, -1e300]))
    assert list(got) == [0x7FC0, 0x7F80, 0xFF80, 0x7F80, 0xFF80]


# ------------------------------------------------------- whole-oracle pins ---

def _golden_gemm():
    cases = []
    a = b = None
    with open(os.path.join(GOLDEN, "handworked_gemm_2x2x2.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("A "):
                a = np.array([int(t, 16) for t in line.split()[1:]], np.uint8).reshape(2, 2)
            elif line.startswith("B "):
                b = np.array([int(t, 16) for t in line.split()[1:]], np.uint8).reshape(2, 2)
            elif line.startswith("case "):
                head, sa, sb, bias, exp = [p.strip() for p in line[5:].split("|")]
                name, mode = head.split()
                cases.append(dict(
                    name=name, mode=int(mode),
                    sa=np.array([float(t) for t in sa.split()], np.float32),
                    sb=np.array([float(t) for t in sb.split()], np.float32),
                    bias=None if bias == "-" else np.array([int(t, 16) for t in bias.split()], np.uint16),
                    exp=np.array([int(t, 16) for t in exp.split()], np.uint16).reshape(2, 2)))
    return a, b, cases


def test_oracle_handworked_example():
    a, b, cases = _golden_gemm()
    assert len(cases) == 3
    for c in cases:
        r = oracle.scaled_mm(a, b, c["sa"], c["sb"], c["bias"], c["mode"])
        assert np.array_equal(r["bits"], c["exp"]), (c["name"], [hex(x) for x in r["bits"].ravel()])


def _torch_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def brute_force(a, b, sa, sb, bias, mode):
    """Exact rational evaluation of the definition: decode with torch's
    e4m3fn (an outside implementation), sum products as Fractions, scale,
    add bias, round once with `_rne_fraction`.  Returns (bits, mag)."""
    da, db = _torch_decode(a), _torch_decode(b)
    M, K = a.shape
    N = b.shape[0]
    bits = np.zeros((M, N), np.uint16)
    mag = np.zeros((M, N), np.float64)
    bias_v = None
    if bias is not None:
        bias_v = torch.from_numpy(bias.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            mg = Fraction(0)
            for k in range(K):
                p = Fraction(float(da[m, k])) * Fraction(float(db[n, k]))
                acc += p
                mg += abs(p)
            if mode == PT:
                s = Fraction(float(sa[0])) * Fraction(float(sb[0]))
            else:
                s = Fraction(float(sa[m])) * Fraction(float(sb[n]))
            y = s * acc
            if bias_v is not None:
                y += Fraction(float(bias_v[n]))
            bits[m, n] = _rne_fraction(y)
            mag[m, n] = float(mg)
    return bits, mag


_NON_NAN = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _tiny_case(seed, M, N, K, mode, with_bias):
    rng = np.random.Generator(np.random.PCG64(seed))
    a = _NON_NAN[rng.integers(0, _NON_NAN.size, (M, K))]
    b = _NON_NAN[rng.integers(0, _NON_NAN.size, (N, K))]
    # a fifth of A's entries are drawn from the smallest codes (zeros and
    # subnormals of both signs) so that those decode paths matter
    small = rng.random((M, K)) < 0.2
    a[small] = rng.integers(0, 16, size=int(small.sum())) | (rng.integers(0, 2, size=int(small.sum())) << 7)
    sa = np.exp2(rng.uniform(-8, 4, M if mode == RW else 1)).astype(np.float32)
    sb = np.exp2(rng.uniform(-8, 4, N if mode == RW else 1)).astype(np.float32)
    bias = None
    if with_bias:
        bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 100).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return a, b, sa, sb, bias


@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 16), (3, 5, 16), (6, 4, 32), (5, 7, 48), (2, 3, 96)])
def test_oracle_equals_exact_brute_force(mode, with_bias, shape):
    M, N, K = shape
    seed = hash((mode, with_bias, shape)) & 0xFFFF
    a, b, sa, sb, bias = _tiny_case(seed, M, N, K, mode, with_bias)
    r = oracle.scaled_mm(a, b, sa, sb, bias, mode)
    bits, mag = brute_force(a, b, sa, sb, bias, mode)
    assert np.array_equal(r["bits"], bits)
    assert np.array_equal(r["mag"], mag)


def _int_units(codes):
    """e4m3fn value in units of 2^-9 as an integer, from the bit fields by a
    different route than the oracle's decode: (8 + m) << (e - 1) for normal
    codes, m for subnormal ones."""
    c = codes.astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return np.where(s == 1, -mag, mag)


def test_acc_is_exact_integer_sum():
    rng = np.random.Generator(np.random.PCG64(3))
    M, N, K = 64, 48, 512
    a = _NON_NAN[rng.integers(0, _NON_NAN.size, (M, K))]
    b = _NON_NAN[rng.integers(0, _NON_NAN.size, (N, K))]
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32))
    ia, ib = _int_units(a), _int_units(b)
    exact = ia @ ib.T                                    # int64, in units of 2^-18
    assert np.array_equal(r["acc"] * 2.0 ** 18, exact.astype(np.float64))
    assert np.array_equal((r["acc"] * 2.0 ** 18).astype(np.int64), exact)
    assert np.array_equal(r["mag"] * 2.0 ** 18, (np.abs(ia) @ np.abs(ib).T).astype(np.float64))


def test_worst_case_magnitude_is_exact():
    """K = 28672 (the largest K of the skinny shapes) with every product at
    the extreme 448 * 448, plus one 2^-9 * 2^-9 term: the sum must keep the
    smallest term."""
    K = 28672
    a = np.full((1, K), 0x7E, np.uint8)
    b = np.full((1, K), 0x7E, np.uint8)
    a[0, 5] = 0x01
    b[0, 5] = 0x01
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32))
    assert Fraction(r["acc"][0, 0]) == (K - 1) * Fraction(448) ** 2 + Fraction(1, 2 ** 18)


# --------------------------------------------------------------- invariants ---

def _normal_case(M, N, K, mode, bias=False, key=0):
    from precision_linear_amd.workloads import make_inputs
    return make_inputs(M, N, K, mode, "normal", bias, key=key)


def test_unit_scales_give_rne_of_acc():
    x = _normal_case(32, 24, 64, PT, key=1)
    one = np.ones(1, np.float32)
    r = oracle.scaled_mm(x.a, x.b, one, one)
    assert np.array_equal(r["bits"], oracle.f64_to_bf16_rne(r["acc"]))


def test_identity_a_reproduces_scaled_b():
    K = 64
    a = np.zeros((K, K), np.uint8)
    a[np.arange(K), np.arange(K)] = 0x38                 # 1.0 on the diagonal
    x = _normal_case(K, 40, K, PT, key=2)
    r = oracle.scaled_mm(a, x.b, np.array([0.75], np.float32), x.scale_b)
    s = 0.75 * float(x.scale_b[0])
    want = oracle.f64_to_bf16_rne(s * _torch_decode(x.b).T)
    assert np.array_equal(r["bits"], want)


def test_one_hot_rows_select_single_products():
    rng = np.random.Generator(np.random.PCG64(5))
    M, N, K = 8, 8, 32
    a = np.zeros((M, K), np.uint8)
    ks = rng.integers(0, K, M)
    a[np.arange(M), ks] = 0x40                           # 2.0
    b = _NON_NAN[rng.integers(0, _NON_NAN.size, (N, K))]
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32))
    want = oracle.f64_to_bf16_rne(2.0 * _torch_decode(b)[:, ks].T)
    # a sum that is zero is +0 even where the one product is -0: compare values
    want = np.where(want == 0x8000, np.uint16(0), want)
    assert np.array_equal(r["bits"], want)


def test_power_of_two_scale_shifts_exponent():
    x = _normal_case(48, 40, 128, PT, key=3)
    r0 = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b)
    r1 = oracle.scaled_mm(x.a, x.b, x.scale_a * np.float32(8.0), x.scale_b)
    v0 = torch.from_numpy(r0["bits"].view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    v1 = torch.from_numpy(r1["bits"].view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(v1, 8.0 * v0)


def test_rowwise_constant_equals_per_tensor():
    x = _normal_case(40, 56, 96, PT, bias=True, key=4)
    M, N = 40, 56
    r_pt = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b, x.bias, PT)
    r_rw = oracle.scaled_mm(x.a, x.b, np.repeat(x.scale_a, M), np.repeat(x.scale_b, N), x.bias, RW)
    assert np.array_equal(r_pt["bits"], r_rw["bits"])


def test_rowwise_scales_pick_row_and_column():
    """Row-wise: out[m, n] must use scale_a[m] and scale_b[n] -- checked by
    making every scale a distinct power of two and comparing with a per-tensor
    call for each (m, n)."""
    M, N, K = 6, 5, 32
    x = _normal_case(M, N, K, RW, key=5)
    sa = np.exp2(np.arange(M, dtype=np.float32) - 3)
    sb = np.exp2(-np.arange(N, dtype=np.float32))
    r = oracle.scaled_mm(x.a, x.b, sa, sb, None, RW)
    for m in range(M):
        for n in range(N):
            p = oracle.scaled_mm(x.a[m:m + 1], x.b[n:n + 1], sa[m:m + 1], sb[n:n + 1], None, PT)
            assert r["bits"][m, n] == p["bits"][0, 0]


def test_zero_a_gives_bias_bits():
    x = _normal_case(16, 64, 32, RW, bias=True, key=6)
    a0 = np.zeros_like(x.a)
    r = oracle.scaled_mm(a0, x.b, x.scale_a, x.scale_b, x.bias, RW)
    assert np.array_equal(r["bits"], np.broadcast_to(x.bias, r["bits"].shape))


def test_sign_flip_negates():
    x = _normal_case(24, 24, 64, PT, key=7)
    r0 = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b)
    r1 = oracle.scaled_mm(x.a ^ np.uint8(0x80), x.b, x.scale_a, x.scale_b)
    nz = (r0["bits"] & 0x7FFF) != 0
    assert np.array_equal(r1["bits"][nz], r0["bits"][nz] ^ np.uint16(0x8000))


def test_zero_k_padding_is_neutral():
    x = _normal_case(20, 30, 48, RW, bias=True, key=8)
    pad_a = np.concatenate([x.a, np.zeros((20, 32), np.uint8)], axis=1)
    pad_b = np.concatenate([x.b, np.full((30, 32), 0x45, np.uint8)], axis=1)
    r0 = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b, x.bias, RW)
    r1 = oracle.scaled_mm(pad_a, pad_b, x.scale_a, x.scale_b, x.bias, RW)
    assert np.array_equal(r0["bits"], r1["bits"])


def test_operand_swap_transposes():
    x = _normal_case(18, 26, 64, PT, key=9)
    r0 = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b)
    r1 = oracle.scaled_mm(x.b, x.a, x.scale_b, x.scale_a)
    assert np.array_equal(r0["bits"], r1["bits"].T)


def test_row_and_column_sampling_matches_full():
    x = _normal_case(33, 29, 80, RW, bias=True, key=10)
    full = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b, x.bias, RW)
    rows, cols = np.array([0, 7, 32]), np.array([28, 3])
    part = oracle.scaled_mm(x.a, x.b, x.scale_a, x.scale_b, x.bias, RW, rows=rows, cols=cols)
    assert np.array_equal(part["bits"], full["bits"][np.ix_(rows, cols)])


def test_nan_code_propagates():
    a = np.full((2, 16), 0x38, np.uint8)
    a[0, 3] = 0x7F
    b = np.full((3, 16), 0x38, np.uint8)
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32))
    assert np.all(r["bits"][0] == 0x7FC0)
    assert np.all(r["bits"][1] == oracle.f64_to_bf16_rne(np.array([16.0]))[0])


def test_nan_times_zero_is_nan():
    # IEEE 754: NaN * 0 is NaN, and a NaN term makes the sum NaN.  The NaN
    # codes here meet only zeros (B's column 3 is zero in every row, A's row 1
    # is zero except a NaN; B's row 2 holds a NaN where A is zero), so a sum
    # that skipped zero products would lose them.
    a = np.full((3, 16), 0x38, np.uint8)
    a[0, 3] = 0x7F
    a[1, :] = 0x00
    a[1, 9] = 0xFF
    a[2, 5] = 0x00
    b = np.full((3, 16), 0x40, np.uint8)
    b[:, 3] = 0x00
    b[:, 9] = 0x00
    b[2, 5] = 0x7F
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32))
    bits = r["bits"]
    assert np.all(bits[0] == 0x7FC0) and np.all(bits[1] == 0x7FC0)
    assert np.all(bits[:, 2] == 0x7FC0)
    # row 2 x columns 0, 1: A[2] = 1.0 except a 0 at k=5, B = 2.0 except zeros
    # at k = 3, 9: 13 products of 2
    assert np.all(bits[2, :2] == oracle.f64_to_bf16_rne(np.array([26.0]))[0])
    # the same with a bias and row-wise scales: NaN stays NaN
    r = oracle.scaled_mm(a, b, np.full(3, 0.5, np.float32), np.full(3, 2.0, np.float32),
                         np.full(3, 0x3F80, np.uint16), RW)
    assert np.all(r["bits"][0] == 0x7FC0) and np.all(r["bits"][:, 2] == 0x7FC0)
    assert np.all(r["bits"][2, :2] == oracle.f64_to_bf16_rne(np.array([27.0]))[0])


# --------------------------------------------------- the pins catch mutants ---

def _mutants():
    """Plausible mistakes planted in copies of the oracle (on the CPU)."""
    good = ref.scaled_mm

    def no_bias(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        return good(a, b, sa, sb, None, mode, rows, cols)

    def scaled_bias(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        r = good(a, b, sa, sb, None, mode, rows, cols)
        if bias is not None:
            y = r["s"] * (r["acc"] + ref.bf16_bits_to_f64(bias)[None, :])
            r = dict(r, bits=ref.f64_to_bf16_rne(y))
        return r

    def swapped_scales(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        if mode == RW and len(sa) == len(sb):
            sa, sb = sb[::-1].copy(), sa[::-1].copy()
        elif mode == RW:
            sa = sa[::-1].copy()
        return good(a, b, sa, sb, bias, mode, rows, cols)

    def truncating_round(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        r = good(a, b, sa, sb, bias, mode, rows, cols)
        t = (r["y"].astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return dict(r, bits=t)

    def via_fp32(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        r = good(a, b, sa, sb, bias, mode, rows, cols)
        f = r["y"].astype(np.float32)
        bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return dict(r, bits=bits)

    def bad_subnormals(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        saved = ref._DECODE.copy()
        ref._DECODE[1:8] = np.arange(1, 8) * 2.0 ** -10
        ref._DECODE[0x81:0x88] = -np.arange(1, 8) * 2.0 ** -10
        try:
            return good(a, b, sa, sb, bias, mode, rows, cols)
        finally:
            ref._DECODE[:] = saved

    def transposed_b(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        if b.shape[0] == b.shape[1]:
            b = np.ascontiguousarray(b.T)
        else:
            b = np.ascontiguousarray(b[::-1])
        return good(a, b, sa, sb, bias, mode, rows, cols)

    def dropped_last_k(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None):
        return good(a[:, :-1], b[:, :-1], sa, sb, bias, mode, rows, cols)

    return dict(no_bias=no_bias, scaled_bias=scaled_bias, swapped_scales=swapped_scales,
                truncating_round=truncating_round, via_fp32=via_fp32,
                bad_subnormals=bad_subnormals, transposed_b=transposed_b,
                dropped_last_k=dropped_last_k)


def _pins_pass(fn) -> bool:
    """A compact re-run of the golden and brute-force pins against `fn`."""
    a, b, cases = _golden_gemm()
    for c in cases:
        if not np.array_equal(fn(a, b, c["sa"], c["sb"], c["bias"], c["mode"])["bits"], c["exp"]):
            return False
    for mode in (PT, RW):
        for with_bias in (False, True):
            for shape in [(3, 5, 16), (4, 4, 32)]:
                M, N, K = shape
                aa, bb, sa, sb, bias = _tiny_case(17 + M * N + mode, M, N, K, mode, with_bias)
                if not np.array_equal(fn(aa, bb, sa, sb, bias, mode)["bits"],
                                      brute_force(aa, bb, sa, sb, bias, mode)[0]):
                    return False
    # double-rounding trap: acc = 16*16 + 1*1 + 2^-9*2^-9 = 257 + 2^-18 lies
    # above the bf16 tie 257 by less than fp32 resolves at 257
    a1 = np.array([[0x58, 0x38, 0x01] + [0] * 13], np.uint8)
    one = np.ones(1, np.float32)
    want = _rne_fraction(Fraction(257) + Fraction(1, 2 ** 18))
    assert want == 0x4381
    if int(fn(a1, a1.copy(), one, one, None, PT)["bits"][0, 0]) != want:
        return False
    return True


def test_pins_accept_the_oracle():
    assert _pins_pass(ref.scaled_mm)


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_pins_reject_planted_mistakes(name):
    assert not _pins_pass(_mutants()[name]), name
