"""Pins for the oracle's e5m2 and mixed-format paths (CPU only).

What fixes them, other than the oracle itself: the OCP e5m2 special values
(golden file), IEEE binary16 (an e5m2 code is the top byte of a binary16
pattern, decoded here by numpy), torch's CPU float8_e5m2 casts (an outside
implementation), exact rational brute force, hand-worked examples, and
invariants; planted mistakes are rejected.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_scaled_mm_ref as ref
from oracle import quantize_ref as qref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PT, RW = oracle.PER_TENSOR, oracle.ROWWISE
E4, E5 = oracle.E4M3FN, oracle.E5M2
FMT = {"e4m3fn": E4, "e5m2": E5}

ALL = np.arange(256, dtype=np.uint8)
E5_FINITE = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)
E4_FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


# ---------------------------------------------------------------- decode ---

def _golden_codes():
    rows = []
    for line in open(os.path.join(GOLDEN, "e5m2_special_codes.txt")):
        line = line.split("#")[0].strip()
        if line:
            code, val = line.split()
            rows.append((int(code, 16), val))
    return rows


def test_decode_golden_special_codes():
    rows = _golden_codes()
    assert len(rows) >= 25
    for code, val in rows:
        got = oracle.e5m2_value(code)
        if val == "nan":
            assert np.isnan(got), hex(code)
        elif val in ("inf", "-inf"):
            assert got == float(val), hex(code)
        else:
            p, q = val.split("/")
            want = Fraction(int(p), int(q))
            assert Fraction(got) == want, hex(code)
            if int(p) == 0:
                assert np.signbit(got) == p.startswith("-"), hex(code)


def test_decode_class_counts():
    v = oracle.e5m2_decode_table()
    assert np.isnan(v).sum() == 6
    assert np.isinf(v).sum() == 2
    fin = v[np.isfinite(v)]
    assert (fin == 0).sum() == 2
    assert ((fin != 0) & (np.abs(fin) < 2.0 ** -14)).sum() == 6      # subnormals
    assert (np.abs(fin) >= 2.0 ** -14).sum() == 240                   # normals
    assert np.nanmax(np.where(np.isinf(v), np.nan, v)) == 57344.0


def test_decode_is_the_top_byte_of_binary16():
    # e5m2 keeps binary16's sign, 5-bit exponent (bias 15) and the top two
    # mantissa bits: code c has the value of the binary16 pattern c << 8.
    half = (ALL.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    got = oracle.decode(ALL, E5)
    assert np.array_equal(np.isnan(got), np.isnan(half))
    ok = ~np.isnan(half)
    assert np.array_equal(got[ok], half[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(half[ok]))


def test_decode_matches_torch_cpu_cast():
    t = torch.from_numpy(ALL.copy()).view(torch.float8_e5m2).to(torch.float64).numpy()
    got = oracle.decode(ALL, E5)
    assert np.array_equal(np.isnan(got), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(got[ok], t[ok])


def test_decode_monotone_symmetric():
    v = oracle.decode(np.arange(0x7C, dtype=np.uint8), E5)          # +0 .. 57344
    assert np.all(np.diff(v) > 0)
    neg = oracle.decode(np.arange(0x80, 0xFC, dtype=np.uint8), E5)
    assert np.array_equal(neg, -v)
    assert oracle.e5m2_value(0x03) + 2.0 ** -16 == oracle.e5m2_value(0x04)


def test_unknown_format_rejected():
    with pytest.raises(ValueError):
        oracle.decode(ALL, 7)


# ---------------------------------------------------------------- encode ---

def test_encode_roundtrips_every_finite_code():
    assert np.array_equal(oracle.encode_rne(oracle.decode(E5_FINITE, E5), E5), E5_FINITE)


def test_encode_equals_integer_rne_of_binary16():
    """For every finite binary16 value up to 57344 in magnitude, RNE to e5m2
    is dropping the low byte of its pattern with round-half-even done on the
    integer (the carry runs into the exponent at binade ends, and the
    subnormals line up because both formats share exponent bias 15)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    val = bits.view(np.float16).astype(np.float64)
    keep = np.isfinite(val) & (np.abs(val) <= 57344.0)
    bits, val = bits[keep], val[keep]
    mag = (bits & 0x7FFF).astype(np.int64)
    r = (mag + 0x7F + ((mag >> 8) & 1)) >> 8
    want = (r | ((bits >> 15).astype(np.int64) << 7)).astype(np.uint8)
    assert np.array_equal(oracle.encode_rne(val, E5), want)


def _nearest_code_e5(y: Fraction) -> int:
    best = None
    for c in range(0x7C):
        d = abs(abs(y) - Fraction(oracle.e5m2_value(c)))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if y < 0 else 0)


def test_encode_matches_rational_brute_force_on_fp32_values():
    rng = np.random.default_rng(11)
    y = (rng.uniform(-1, 1, 400) * np.exp2(rng.integers(-20, 16, 400))).astype(np.float32)
    y = np.clip(y, -57344, 57344)
    got = oracle.encode_rne(y.astype(np.float64), E5)
    for v, g in zip(y, got):
        if v == 0:
            continue
        assert g == _nearest_code_e5(Fraction(float(v))), float(v)


def test_encode_matches_torch_cpu_cast():
    rng = np.random.default_rng(12)
    y = (rng.uniform(-1, 1, 300000) * np.exp2(rng.integers(-20, 16, 300000))).astype(np.float32)
    y = np.clip(y, -57344, 57344)
    want = torch.from_numpy(y).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_rne(y.astype(np.float64), E5), want)


def test_encode_rejects_unclamped():
    with pytest.raises(ValueError):
        oracle.encode_rne(np.array([57345.0]), E5)


# ------------------------------------------------------------ scaled multiply ---

def _golden_gemm():
    cases = []
    for line in open(os.path.join(GOLDEN, "handworked_e5m2_gemm.txt")):
        line = line.split("#")[0].strip()
        if not line.startswith("case "):
            continue
        head, a, b, mode, sa, sb, bias, exp = [p.strip() for p in line[5:].split("|")]
        name, fa, fb, M, N, K = head.split()
        M, N, K = int(M), int(N), int(K)
        cases.append(dict(
            name=name, fa=FMT[fa], fb=FMT[fb], mode=int(mode),
            a=np.array([int(t, 16) for t in a.split()], np.uint8).reshape(M, K),
            b=np.array([int(t, 16) for t in b.split()], np.uint8).reshape(N, K),
            sa=np.array([float(t) for t in sa.split()], np.float32),
            sb=np.array([float(t) for t in sb.split()], np.float32),
            bias=None if bias == "-" else np.array([int(t, 16) for t in bias.split()], np.uint16),
            exp=np.array([int(t, 16) for t in exp.split()], np.uint16).reshape(M, N)))
    return cases


def test_handworked_examples():
    cases = _golden_gemm()
    assert len(cases) == 4
    for c in cases:
        r = oracle.scaled_mm(c["a"], c["b"], c["sa"], c["sb"], c["bias"], c["mode"],
                             a_format=c["fa"], b_format=c["fb"])
        assert np.array_equal(r["bits"], c["exp"]), (c["name"], [hex(x) for x in r["bits"].ravel()])
    cancel = cases[0]
    r = oracle.scaled_mm(cancel["a"], cancel["b"], cancel["sa"], cancel["sb"], None, PT,
                         a_format=E5, b_format=E5)
    assert r["acc"][0, 0] == 2.0 ** -32


def _torch_decode(codes, fmt):
    dt = torch.float8_e4m3fn if fmt == E4 else torch.float8_e5m2
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(dt).to(torch.float64).numpy()


def _rne_bf16(y: Fraction) -> int:
    from test_oracle_pins import _rne_fraction
    return _rne_fraction(y)


def brute_force(a, b, sa, sb, bias, mode, fa, fb):
    """Exact rationals from torch's decode: (bits, exact acc as Fractions)."""
    da, db = _torch_decode(a, fa), _torch_decode(b, fb)
    M, K = a.shape
    N = b.shape[0]
    bits = np.zeros((M, N), np.uint16)
    accs = [[None] * N for _ in range(M)]
    bias_v = None
    if bias is not None:
        bias_v = torch.from_numpy(bias.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    for m in range(M):
        for n in range(N):
            acc = sum((Fraction(float(da[m, k])) * Fraction(float(db[n, k])) for k in range(K)),
                      Fraction(0))
            accs[m][n] = acc
            s = Fraction(float(sa[0 if mode == PT else m])) * Fraction(float(sb[0 if mode == PT else n]))
            y = s * acc
            if bias_v is not None:
                y += Fraction(float(bias_v[n]))
            bits[m, n] = _rne_bf16(y)
    return bits, accs


def _tiny_case(seed, M, N, K, mode, with_bias, fa, fb):
    rng = np.random.Generator(np.random.PCG64(seed))
    pool = {E4: E4_FINITE, E5: E5_FINITE}
    a = pool[fa][rng.integers(0, pool[fa].size, (M, K))]
    b = pool[fb][rng.integers(0, pool[fb].size, (N, K))]
    # a fifth of the entries come from the smallest codes (zeros, subnormals)
    for x, f in ((a, fa), (b, fb)):
        small = rng.random(x.shape) < 0.2
        lim = 16 if f == E4 else 8
        x[small] = rng.integers(0, lim, size=int(small.sum())) | (rng.integers(0, 2, size=int(small.sum())) << 7)
    sa = np.exp2(rng.uniform(-8, 4, M if mode == RW else 1)).astype(np.float32)
    sb = np.exp2(rng.uniform(-8, 4, N if mode == RW else 1)).astype(np.float32)
    bias = None
    if with_bias:
        bias = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * 100).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return a, b, sa, sb, bias


FORMAT_PAIRS = [(E5, E5), (E4, E5), (E5, E4)]


@pytest.mark.parametrize("fa,fb", FORMAT_PAIRS)
@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 16), (3, 5, 16), (4, 3, 48)])
def test_oracle_equals_exact_brute_force(fa, fb, mode, with_bias, shape):
    M, N, K = shape
    seed = (fa * 7 + fb * 3 + mode * 11 + with_bias * 13 + M * 17 + K) & 0xFFFF
    a, b, sa, sb, bias = _tiny_case(seed, M, N, K, mode, with_bias, fa, fb)
    r = oracle.scaled_mm(a, b, sa, sb, bias, mode, a_format=fa, b_format=fb)
    bits, accs = brute_force(a, b, sa, sb, bias, mode, fa, fb)
    assert np.array_equal(r["bits"], bits)
    for m in range(M):
        for n in range(N):
            assert r["acc"][m, n] == float(accs[m][n])      # the exact sum rounded once


def _int_units(codes, fmt):
    """Value in units of the format's smallest subnormal, from the bit fields
    by another route than the decode table: (2^mb + m) << (e - 1) for normal
    codes, m for subnormal ones."""
    mb = 3 if fmt == E4 else 2
    c = codes.astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> mb) & ((1 << (7 - mb)) - 1)
    m = c & ((1 << mb) - 1)
    mag = np.where(e == 0, m, ((1 << mb) + m) << np.maximum(e - 1, 0))
    return np.where(s == 1, -mag, mag)


@pytest.mark.parametrize("fa,fb", FORMAT_PAIRS)
def test_acc_is_the_exact_integer_sum_rounded_once(fa, fb):
    rng = np.random.Generator(np.random.PCG64(5 + fa + 2 * fb))
    M, N, K = 24, 20, 256
    pool = {E4: E4_FINITE, E5: E5_FINITE}
    a = pool[fa][rng.integers(0, pool[fa].size, (M, K))]
    b = pool[fb][rng.integers(0, pool[fb].size, (N, K))]
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32), a_format=fa, b_format=fb)
    ia, ib = _int_units(a, fa), _int_units(b, fb)
    q = oracle.UNIT_EXP[fa] + oracle.UNIT_EXP[fb]
    for m in range(M):
        for n in range(N):
            exact = sum(int(x) * int(y) for x, y in zip(ia[m], ib[n]))
            assert r["acc"][m, n] == float(Fraction(exact, 1 << q))


def test_extreme_span_at_largest_k():
    """K = 28672 with every product at 57344^2 except one 2^-16 * 2^-16 term
    and one that cancels a big one: the sum must keep the smallest term."""
    K = 28672
    a = np.full((1, K), 0x7B, np.uint8)
    b = np.full((1, K), 0x7B, np.uint8)
    a[0, 5] = b[0, 5] = 0x01
    b[0, 9] = 0xFB
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32), a_format=E5, b_format=E5)
    exact = (K - 3) * Fraction(57344) ** 2 + Fraction(1, 2 ** 32)
    assert r["acc"][0, 0] == float(exact)
    # and the cancellation alone, where fp64 summation would lose the small term
    a2 = np.array([[0x7B, 0x01, 0x7B] + [0] * 13], np.uint8)
    b2 = np.array([[0x7B, 0x01, 0xFB] + [0] * 13], np.uint8)
    r2 = oracle.scaled_mm(a2, b2, np.ones(1, np.float32), np.ones(1, np.float32), a_format=E5, b_format=E5)
    assert r2["acc"][0, 0] == 2.0 ** -32


# Non-finite e5m2 codes: +inf 0x7C, -inf 0xFC, NaN 0x7D..0x7F and 0xFD..0xFF.
# Each case is one row of A against one row of B (K = 16, the rest zeros),
# with the IEEE 754 result written out by hand: inf times zero is NaN, a NaN
# factor or term gives NaN, +inf and -inf terms together give NaN, and a lone
# infinity keeps the sign of its factors' signs' product.
INF, NINF, NAN, ONE, TWO, MONE, MTWO, ZERO, MZERO = 0x7C, 0xFC, 0x7D, 0x3C, 0x40, 0xBC, 0xC0, 0x00, 0x80
NONFINITE_CASES = [
    ([INF, ONE], [ONE, ONE], 0x7F80),        # inf + 1 = inf
    ([INF, ONE], [MONE, ONE], 0xFF80),       # -inf + 1 = -inf
    ([NINF], [MTWO], 0x7F80),                # (-inf)(-2) = inf
    ([INF, INF], [ONE, TWO], 0x7F80),        # inf + inf = inf
    ([INF, ONE], [ZERO, ONE], None),         # inf * 0 = NaN
    ([INF, ONE], [MZERO, ONE], None),        # inf * -0 = NaN
    ([ZERO, TWO], [NINF, ONE], None),        # 0 * -inf = NaN
    ([INF, NINF], [ONE, ONE], None),         # inf - inf = NaN
    ([INF, ONE], [ONE, NINF], None),         # inf + (-inf) = NaN
    ([0x7F, ONE], [ZERO, ONE], None),        # NaN * 0 = NaN
    ([ONE, ONE], [0xFE, ONE], None),         # NaN term
    ([ONE, TWO], [ONE, ONE], 0x4040),        # finite: 1 + 2 = 3 (bf16 0x4040)
]


@pytest.mark.parametrize("ca,cb,want", NONFINITE_CASES)
def test_nonfinite_e5m2_follow_ieee(ca, cb, want):
    a = np.zeros((1, 16), np.uint8)
    b = np.zeros((1, 16), np.uint8)
    a[0, :len(ca)] = ca
    b[0, :len(cb)] = cb
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32), a_format=E5, b_format=E5)
    got = int(r["bits"][0, 0])
    if want is None:
        assert np.isnan(r["acc"][0, 0]) and got == 0x7FC0
    else:
        assert got == want, hex(got)


@pytest.mark.parametrize("cb,want", [([0x38, 0x38], 0x7F80),     # e4m3fn 1, 1: inf + 1
                                     ([0x00, 0x38], None),       # e4m3fn 0: inf * 0
                                     ([0xB8, 0x38], 0xFF80),     # e4m3fn -1: -inf + 1
                                     ([0x7F, 0x38], None)])      # e4m3fn NaN
def test_nonfinite_e5m2_times_e4m3fn(cb, want):
    a = np.array([[INF, ONE] + [0] * 14], np.uint8)
    b = np.array([cb + [0] * 14], np.uint8)
    r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32), a_format=E5, b_format=E4)
    got = int(r["bits"][0, 0])
    if want is None:
        assert got == 0x7FC0
    else:
        assert got == want, hex(got)


def test_nonfinite_e5m2_scale_zero_and_bias():
    # 0 * inf = NaN after the scale; inf + bias = inf
    a = np.array([[INF] + [0] * 15], np.uint8)
    b = np.array([[ONE] + [0] * 15], np.uint8)
    r0 = oracle.scaled_mm(a, b, np.zeros(1, np.float32), np.ones(1, np.float32), a_format=E5, b_format=E5)
    assert r0["bits"][0, 0] == 0x7FC0
    bias = np.array([0xC2C8], np.uint16)            # bf16 -100
    r1 = oracle.scaled_mm(a, b, np.full(1, 0.5, np.float32), np.ones(1, np.float32), bias,
                          a_format=E5, b_format=E5)
    assert r1["bits"][0, 0] == 0x7F80


def _binary16_value(code):
    """An e5m2 code is the top byte of an IEEE binary16 pattern."""
    return float(np.array([int(code) << 8], np.uint16).view(np.float16)[0])


def test_nonfinite_e5m2_against_python_floats():
    """Random small matrices with sparse inf / NaN codes and zeros: the
    oracle's acc against a plain Python loop in IEEE doubles over values
    decoded as binary16 (infinities and NaNs propagate by the hardware's own
    IEEE rules there).  Non-finite results must agree exactly (NaN, or the
    same infinity); finite ones equal the exact sum of the products
    (fractions.Fraction) rounded once to double."""
    rng = np.random.default_rng(17)
    M, N, K = 9, 7, 32
    pool = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], np.uint8)     # finite codes

    def draw(rows):
        x = pool[rng.integers(0, pool.size, (rows, K))]
        x[rng.random((rows, K)) < 0.15] = 0
        special = rng.random((rows, K)) < 0.05
        x[special] = rng.choice(np.array([0x7C, 0xFC, 0x7D, 0xFF], np.uint8), special.sum())
        return x

    for trial in range(6):
        a, b = draw(M), draw(N)
        r = oracle.scaled_mm(a, b, np.ones(1, np.float32), np.ones(1, np.float32), a_format=E5, b_format=E5)
        for m in range(M):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += _binary16_value(a[m, k]) * _binary16_value(b[n, k])
                got = r["acc"][m, n]
                if np.isnan(acc):
                    assert np.isnan(got), (trial, m, n)
                elif np.isinf(acc):
                    assert got == acc, (trial, m, n, got, acc)
                else:
                    exact = sum(Fraction(_binary16_value(a[m, k])) * Fraction(_binary16_value(b[n, k]))
                                for k in range(K))
                    assert got == float(exact), (trial, m, n)


# ---------------------------------------------------------------- invariants ---

def test_e4m3_values_recoded_as_e5m2_give_the_same_output():
    """e4m3fn codes whose values e5m2 holds exactly (mantissa low bit 0,
    within e5m2's range) give bit-identical results when re-coded."""
    rng = np.random.default_rng(21)
    M, N, K = 6, 5, 64
    ok = np.array([c for c in E4_FINITE if (c & 1) == 0], np.uint8)
    a = ok[rng.integers(0, ok.size, (M, K))]
    b = E4_FINITE[rng.integers(0, E4_FINITE.size, (N, K))]
    a5 = oracle.encode_rne(oracle.decode(a, E4), E5)
    assert np.array_equal(oracle.decode(a5, E5), oracle.decode(a, E4))
    sa = np.exp2(rng.uniform(-4, 4, M)).astype(np.float32)
    sb = np.exp2(rng.uniform(-4, 4, N)).astype(np.float32)
    r4 = oracle.scaled_mm(a, b, sa, sb, None, RW)
    r5 = oracle.scaled_mm(a5, b, sa, sb, None, RW, a_format=E5, b_format=E4)
    assert np.array_equal(r4["bits"], r5["bits"])
    assert np.array_equal(r4["acc"], r5["acc"])


def test_operand_swap_transposes():
    a, b, sa, sb, _ = _tiny_case(3, 5, 4, 32, RW, False, E4, E5)
    r = oracle.scaled_mm(a, b, sa, sb, None, RW, a_format=E4, b_format=E5)
    t = oracle.scaled_mm(b, a, sb, sa, None, RW, a_format=E5, b_format=E4)
    assert np.array_equal(r["bits"], t["bits"].T)


def test_sign_flip_negates():
    a, b, sa, sb, _ = _tiny_case(4, 4, 6, 32, PT, False, E5, E5)
    r = oracle.scaled_mm(a, b, sa, sb, None, PT, a_format=E5, b_format=E5)
    f = oracle.scaled_mm(a ^ np.uint8(0x80), b, sa, sb, None, PT, a_format=E5, b_format=E5)
    assert np.array_equal(f["bits"], r["bits"] ^ np.uint16(0x8000))


# ------------------------------------------------------------ quantiser (e5m2) ---

def to_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _golden_quant():
    x, rs, rc, ps, pc = [], None, [], None, []
    for line in open(os.path.join(GOLDEN, "quantize_e5m2_handworked.txt")):
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


def test_quantize_handworked_example():
    x, rs, rc, ps, pc = _golden_quant()
    xb = to_bf16_bits(x)
    assert np.array_equal(oracle.bf16_bits_to_f64(xb), x.astype(np.float64))
    q, s = oracle.quantize(xb, RW, E5)
    assert np.array_equal(s.view(np.uint32), rs) and np.array_equal(q, rc)
    q, s = oracle.quantize(xb, PT, E5)
    assert np.array_equal(s.view(np.uint32), ps) and np.array_equal(q, pc)


@pytest.mark.parametrize("mode", [PT, RW])
def test_quantize_matches_torch_recipe(mode):
    """torch's own ops, step by step as the gist writes them, on bf16 data."""
    rng = np.random.default_rng(31 + mode)
    x = (rng.standard_normal((40, 300)) * np.exp2(rng.integers(-12, 12, (40, 1)))).astype(np.float32)
    x[3] = 0.0
    xb = to_bf16_bits(x)
    t = torch.from_numpy(xb.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32)
    amax = t.abs().amax(dim=1, keepdim=True) if mode == RW else t.abs().amax().reshape(1, 1)
    scale = amax / torch.tensor(57344.0)
    y = torch.where(scale > 0, t / torch.where(scale > 0, scale, torch.ones_like(scale)), torch.zeros_like(t))
    want = y.clamp(-57344.0, 57344.0).to(torch.float8_e5m2).view(torch.uint8).numpy()
    q, s = oracle.quantize(xb, mode, E5)
    assert np.array_equal(q, want)
    assert np.array_equal(s, scale.reshape(-1).numpy())


def test_quantize_row_max_maps_to_57344():
    rng = np.random.default_rng(7)
    xb = to_bf16_bits(rng.standard_normal((16, 129)).astype(np.float32))
    q, s = oracle.quantize(xb, RW, E5)
    x = oracle.bf16_bits_to_f64(xb)
    j = np.argmax(np.abs(x), axis=1)
    assert np.all((q[np.arange(16), j] & 0x7F) == 0x7B)


def test_quantize_dequantised_error_within_half_e5m2_spacing():
    rng = np.random.default_rng(8)
    xb = to_bf16_bits(rng.standard_normal((24, 512)).astype(np.float32) * 3)
    x = oracle.bf16_bits_to_f64(xb)
    q, s = oracle.quantize(xb, RW, E5)
    d = oracle.dequantize(q, s, RW, E5)
    y = x / s.astype(np.float64)[:, None]
    a = np.abs(y)
    _, e = np.frexp(a)
    spacing = np.where(a >= 2.0 ** -14, np.ldexp(1.0, e - 3), 2.0 ** -16)
    bound = (0.5 * spacing + a * 2.0 ** -23) * s.astype(np.float64)[:, None]
    assert np.all(np.abs(d - x) <= bound)


# ------------------------------------------------- the pins catch mutants ---

def _pins_pass(scaled_mm, quantize) -> bool:
    for c in _golden_gemm():
        r = scaled_mm(c["a"], c["b"], c["sa"], c["sb"], c["bias"], c["mode"], a_format=c["fa"], b_format=c["fb"])
        if not np.array_equal(r["bits"], c["exp"]):
            return False
    for fa, fb in FORMAT_PAIRS:
        for mode in (PT, RW):
            a, b, sa, sb, bias = _tiny_case(40 + fa + 2 * fb + 4 * mode, 3, 4, 32, mode, mode == RW, fa, fb)
            if not np.array_equal(scaled_mm(a, b, sa, sb, bias, mode, a_format=fa, b_format=fb)["bits"],
                                  brute_force(a, b, sa, sb, bias, mode, fa, fb)[0]):
                return False
    x, rs, rc, ps, pc = _golden_quant()
    q, s = quantize(to_bf16_bits(x), RW, E5)
    return np.array_equal(q, rc) and np.array_equal(s.view(np.uint32), rs)


def _mutants():
    good_mm, good_q = ref.scaled_mm, qref.quantize

    def fp64_sum(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None, a_format=E4, b_format=E4):
        # the e4m3 path's plain fp64 product for every format (loses cancellations)
        saved = ref._exact_integer_acc
        ref._exact_integer_acc = lambda da, db, qa, qb: da @ db.T
        try:
            return good_mm(a, b, sa, sb, bias, mode, rows, cols, a_format, b_format)
        finally:
            ref._exact_integer_acc = saved

    def e5_bias_16(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None, a_format=E4, b_format=E4):
        saved = ref._DECODE_E5M2.copy()
        ref._DECODE_E5M2[:] = saved * 0.5
        try:
            return good_mm(a, b, sa, sb, bias, mode, rows, cols, a_format, b_format)
        finally:
            ref._DECODE_E5M2[:] = saved

    def swapped_formats(a, b, sa, sb, bias=None, mode=PT, rows=None, cols=None, a_format=E4, b_format=E4):
        return good_mm(a, b, sa, sb, bias, mode, rows, cols, b_format, a_format)

    def e4m3_limit(x_bits, mode=RW, fmt=E4):
        q, s = good_q(x_bits, mode, E4 if fmt == E5 else fmt)
        return q, s

    def truncating_encode(x_bits, mode=RW, fmt=E4):
        saved = qref.np.rint
        qref.np.rint = np.trunc
        try:
            return good_q(x_bits, mode, fmt)
        finally:
            qref.np.rint = saved

    return {"fp64_sum": (fp64_sum, good_q), "e5_bias_16": (e5_bias_16, good_q),
            "swapped_formats": (swapped_formats, good_q), "e4m3_limit": (good_mm, e4m3_limit),
            "truncating_encode": (good_mm, truncating_encode)}


def test_pins_accept_the_oracle():
    assert _pins_pass(ref.scaled_mm, qref.quantize)


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_pins_reject_planted_mistakes(name):
    mm, q = _mutants()[name]
    assert not _pins_pass(mm, q), name
