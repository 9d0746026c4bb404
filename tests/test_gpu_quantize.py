"""GPU parity of the dynamic float8 quantisers (fp8_quantize_e4m3 and
fp8_quantize_e5m2, through the C ABI via the ctypes binding) against the CPU
oracle: codes and scales bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from precision_linear_amd import binding
from parity import compare

pytestmark = pytest.mark.gpu
PT, RW = oracle.PER_TENSOR, oracle.ROWWISE
DEV = "cuda:0"
FMTS = ["e4m3fn", "e5m2"]
OFMT = {"e4m3fn": oracle.E4M3FN, "e5m2": oracle.E5M2}
QMAX = {"e4m3fn": 448.0, "e5m2": 57344.0}


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run(bits, mode, fmt="e4m3fn"):
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    print(f"[quantize] shape={bits.shape} mode={mode} fmt={fmt}", flush=True)
    q, s = binding.fp8_quantize(x, mode, fmt=fmt)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check(bits, mode, fmt="e4m3fn"):
    q, s = run(bits, mode, fmt)
    rq, rs = oracle.quantize(bits, mode, OFMT[fmt])
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), "scales differ"
    bad = np.argwhere(q != rq)
    assert bad.size == 0, (f"{len(bad)} codes differ, first at {tuple(bad[0])}: "
                           f"got {q[tuple(bad[0])]:#04x} want {rq[tuple(bad[0])]:#04x}")
    return q, s


def _normal(rows, cols, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    if spread:
        x *= np.exp2(rng.integers(-30, 30, (rows, 1))).astype(np.float32)
    return bf16_bits(x)


# cols: one 4096-element chunk, a ragged second chunk, the register-resident
# 7-8 chunks (28672) and a row too long for registers (40960)
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (37, 4096), (19, 4112), (8, 16384),
                                       (5, 28672), (3, 40960), (300, 272)])
def test_random_matrices_bitexact(rows, cols, mode, fmt):
    check(_normal(rows, cols, rows * 7 + cols), mode, fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_every_in_range_bf16_value_converts_like_the_oracle(fmt):
    # per-tensor amax = qmax gives scale 1, so y = x: every bf16 value in
    # [-qmax, qmax] (ties, subnormals, -0) goes through the conversion as is
    allb = np.arange(65536, dtype=np.uint32)
    v = (allb << 16).view(np.float32)
    keep = np.isfinite(v) & (np.abs(v) <= QMAX[fmt])
    bits = allb[keep].astype(np.uint16)
    pad = bf16_bits([QMAX[fmt]])[0]
    bits = np.concatenate([bits, np.full((-len(bits)) % 16, pad, np.uint16)])   # pad with qmax
    q, s = check(bits.reshape(-1, 16), PT, fmt)
    assert s[0] == 1.0


@pytest.mark.parametrize("fmt", FMTS)
def test_every_finite_bf16_value_with_a_huge_amax(fmt):
    # amax = the largest bf16: x/s spans underflow to zero, subnormals and qmax
    allb = np.arange(65536, dtype=np.uint32)
    v = (allb << 16).view(np.float32)
    bits = allb[np.isfinite(v)].astype(np.uint16)
    bits = np.concatenate([bits, np.zeros((-len(bits)) % 16, np.uint16)])
    check(bits.reshape(-1, 16), PT, fmt)
    check(bits.reshape(-1, 256), RW, fmt)


def _rows_below_amax(amax_bits, cols, seed):
    """Row r: amax_bits[r] itself, then random bf16 values of either sign whose
    magnitude patterns are drawn uniformly from [0, amax_bits[r]] (so the row's
    amax is exactly that value and x / scale sweeps every binade below it,
    subnormals included)."""
    rng = np.random.default_rng(seed)
    out = np.empty((len(amax_bits), cols), np.uint16)
    for r, a in enumerate(amax_bits):
        mag = rng.integers(0, int(a) + 1, cols).astype(np.uint16)
        sign = rng.integers(0, 2, cols).astype(np.uint16) << 15
        out[r] = mag | sign
        out[r, 0] = a
    return out


@pytest.mark.parametrize("cols", [8192, 65536])    # rows held in registers / read twice
@pytest.mark.parametrize("fmt", FMTS)
def test_division_over_the_scale_range(fmt, cols):
    # x / scale must be the correctly rounded fp32 quotient for the codes to
    # match: amax values across the whole positive finite bf16 range (scales
    # from subnormal to ~2^119), densest around the 2^-60 scale at which the
    # kernel changes its division method, each with a row of values below it
    qmax = QMAX[fmt]
    edge = int(bf16_bits([2.0 ** -60 * qmax])[0])
    amax = np.unique(np.concatenate([
        np.linspace(1, 0x7F7F, 40).astype(np.int64),
        np.arange(edge - 12, edge + 13),
        bf16_bits([1.0, qmax, 3.0e38, 1e-38, 2.0 ** -126]).astype(np.int64)])).astype(np.uint16)
    rows = 24 if cols == 65536 else len(amax)
    sel = amax if rows == len(amax) else amax[np.linspace(0, len(amax) - 1, rows).astype(int)]
    bits = _rows_below_amax(sel, cols, seed=cols + len(fmt))
    check(bits, RW, fmt)
    for a in (sel[0], edge, sel[-1]):     # per-tensor: one scale for the whole matrix
        check(_rows_below_amax(np.full(4, a, np.uint16), 4096, seed=int(a)), PT, fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode", [PT, RW])
def test_nan_elements_give_nan_codes(fmt, mode):
    # outside the finite-input contract: the amax skips a NaN, which comes out
    # as a NaN code (as through torch's clamp); every other element is
    # quantised as if the NaN were 0 (which leaves each amax unchanged)
    bits = _normal(6, 4096, 21)
    nan_pos = [(0, 5), (2, 4095), (3, 0), (3, 1), (5, 2048)]
    for r, c in nan_pos:
        bits[r, c] = 0x7FC0 if c % 2 == 0 else 0xFFC0
    q, s = run(bits, mode, fmt)
    clean = bits.copy()
    for r, c in nan_pos:
        clean[r, c] = 0
    rq, rs = oracle.quantize(clean, mode, OFMT[fmt])
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32))
    mask = np.ones(bits.shape, bool)
    for r, c in nan_pos:
        mask[r, c] = False
        code = int(q[r, c]) & 0x7F
        assert (code == 0x7F) if fmt == "e4m3fn" else (code > 0x7C), hex(q[r, c])
    assert np.array_equal(q[mask], rq[mask])


def test_e5m2_zero_rows_and_signed_zeros():
    x = np.array(_normal(6, 64, 3).view(np.int16), np.int16).view(np.uint16).copy()
    x[1] = 0x0000
    x[2] = 0x8000
    x[3, 5] = 0x8000
    x[4] = 0
    x[4, 7] = bf16_bits([[-3.0]])[0, 0]
    q, s = check(x, RW, "e5m2")
    assert s[1] == 0 and s[2] == 0 and np.all(q[1] == 0) and np.all(q[2] == 0)
    assert q[4, 7] == 0xFB and q[3, 5] == 0x80


def test_zero_rows_and_signed_zeros():
    x = np.array(_normal(6, 64, 3).view(np.int16), np.int16).view(np.uint16).copy()
    x[1] = 0x0000            # all +0
    x[2] = 0x8000            # all -0
    x[3, 5] = 0x8000         # a -0 in a normal row
    x[4] = 0
    x[4, 7] = bf16_bits([[-3.0]])[0, 0]
    q, s = check(x, RW)
    assert s[1] == 0 and s[2] == 0 and np.all(q[1] == 0) and np.all(q[2] == 0)
    assert q[4, 7] == 0xFE and q[3, 5] == 0x80
    check(np.zeros((4, 32), np.uint16), PT)


@pytest.mark.parametrize("mode", [PT, RW])
def test_empty(mode):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    q, s = binding.fp8_quantize(x, mode)
    torch.cuda.synchronize()
    assert q.numel() == 0 and s.numel() == (1 if mode == PT else 0)
    if mode == PT:
        assert s.item() == 0.0
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    sc = torch.full((1 if mode == PT else 5,), 7.0, device=DEV)
    q, s = binding.fp8_quantize(x, mode, scale=sc)
    torch.cuda.synchronize()
    assert torch.all(s == 0)


def test_repeated_calls_are_identical():
    bits = _normal(64, 4096, 11)
    a = run(bits, PT)
    b = run(bits, PT)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("fa,fb", [("e4m3fn", "e4m3fn"), ("e5m2", "e5m2"), ("e4m3fn", "e5m2")])
@pytest.mark.parametrize("mode", [PT, RW])
def test_quantize_then_multiply(mode, fa, fb):
    # the quantiser's outputs are the multiply's inputs: A (M x K) and B (N x K)
    M, N, K = 96, 160, 512
    xa, xb = _normal(M, K, 21, spread=False), _normal(N, K, 22, spread=False)
    ta = torch.from_numpy(xa.view(np.int16)).view(torch.bfloat16).to(DEV)
    tb = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(DEV)
    qa, sa = binding.fp8_quantize(ta, mode, fmt=fa)
    qb, sb = binding.fp8_quantize(tb, mode, fmt=fb)
    out = binding.fp8_scaled_mm(qa, qb, sa, sb, mode=mode, a_format=fa, b_format=fb)
    torch.cuda.synchronize()
    ra, rsa = oracle.quantize(xa, mode, OFMT[fa])
    rb, rsb = oracle.quantize(xb, mode, OFMT[fb])
    assert np.array_equal(qa.cpu().numpy(), ra) and np.array_equal(qb.cpu().numpy(), rb)
    ref = oracle.scaled_mm(ra, rb, rsa, rsb, None, mode, a_format=OFMT[fa], b_format=OFMT[fb])
    nbad, worst, first = compare(out.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    assert nbad == 0, (nbad, worst, first)


def test_outputs_on_another_device_are_refused():
    x = torch.from_numpy(_normal(8, 64, 4).view(np.int16)).view(torch.bfloat16).to(DEV)
    with pytest.raises(ValueError):
        binding.fp8_quantize(x, RW, q=torch.empty(8, 64, dtype=torch.uint8))
    with pytest.raises(ValueError):
        binding.fp8_quantize(x, PT, scale=torch.empty(1, dtype=torch.float32))
    q, s = binding.fp8_quantize(x, RW)
    torch.cuda.synchronize()
    assert q.is_cuda and s.is_cuda


# ------------------------------------------------- the large-input code paths ---

def _workload_bits(rows, cols, key):
    from precision_linear_amd import workloads as wl
    return wl.bf16_matrix_bits(rows, cols, key=key)


@pytest.mark.parametrize("rows,cols,fmt", [(8192, 8192, "e4m3fn"), (8192, 8192, "e5m2"),
                                           (8192, 4096, "e4m3fn"), (4099, 8192, "e4m3fn")])
def test_per_tensor_large_bitexact(rows, cols, fmt):
    # The benchmarked per-tensor size and the sizes around it: the amax and
    # quantisation passes run their unrolled grid-stride loops (every
    # workgroup takes several strides), and the scale comes from the maxima of
    # the whole grid of workgroups (2048 on 256 CUs).  The matrix's amax is
    # planted in the last elements, which the last stride of the last
    # workgroups reads.
    bits = _workload_bits(rows, cols, key=rows + cols + len(fmt))
    bits[-1, -1] = bf16_bits([-9.5])[0]
    check(bits, PT, fmt)


@pytest.mark.parametrize("rows,cols,fmt", [(40000, 256, "e4m3fn"), (40000, 256, "e5m2"),
                                           (33000, 4112, "e4m3fn")])
def test_rowwise_more_rows_than_workgroups_bitexact(rows, cols, fmt):
    # More rows than the row-wise grid (128 workgroups per CU): workgroups
    # walk several rows with the next row prefetched into registers.
    bits = _workload_bits(rows, cols, key=rows * 3 + cols + len(fmt))
    check(bits, RW, fmt)
