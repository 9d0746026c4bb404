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


def run(bits, mode, fmt="e4m3fn", workspace=True):
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    print(f"[quantize] shape={bits.shape} mode={mode} fmt={fmt} workspace={workspace}", flush=True)
    q, s = binding.fp8_quantize(x, mode, fmt=fmt, workspace=workspace)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def check(bits, mode, fmt="e4m3fn", workspace=True):
    q, s = run(bits, mode, fmt, workspace)
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
# mode and path: per-tensor with a workspace (these shapes are below the
# one-pass kernel's size threshold, so this checks that the selection falls
# back to the two-pass kernels) and without one; row-wise uses no workspace.
# The one-pass kernel itself is checked at the sizes that take it, below.
PATHS = [(PT, True), (PT, False), (RW, True)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mode,workspace", PATHS)
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (37, 4096), (19, 4112), (8, 16384),
                                       (5, 28672), (3, 40960), (300, 272)])
def test_random_matrices_bitexact(rows, cols, mode, workspace, fmt):
    check(_normal(rows, cols, rows * 7 + cols), mode, fmt, workspace)


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


@pytest.mark.parametrize("workspace", [True, False], ids=["onepass", "twopass"])
@pytest.mark.parametrize("rows,cols,fmt", [(8192, 8192, "e4m3fn"), (8192, 8192, "e5m2"),
                                           (8192, 4096, "e4m3fn"), (4099, 8192, "e4m3fn"),
                                           (6000, 8192, "e5m2")])
def test_per_tensor_large_bitexact(rows, cols, fmt, workspace):
    # The benchmarked per-tensor size and the sizes around it.  Two passes:
    # the amax and quantisation passes run their unrolled grid-stride loops
    # (every workgroup takes several strides), and the scale comes from the
    # maxima of the whole grid of workgroups (2048 on 256 CUs).  One pass, with
    # 256 workgroups of 1024 groups per step: 8192 x 4096 and 4099 x 8192 are
    # 8 steps (all held in registers), 6000 x 8192 12 (registers, then part
    # of the first LDS step), 8192 x 8192 16 (registers, LDS, and one step
    # read again in the conversion).  The matrix's amax is planted in the
    # last elements, which the last stride of the last workgroups reads.
    bits = _workload_bits(rows, cols, key=rows + cols + len(fmt))
    bits[-1, -1] = bf16_bits([-9.5])[0]
    check(bits, PT, fmt, workspace)


def _quantize_ws():
    stream = torch.cuda.current_stream(torch.device(DEV)).cuda_stream
    return binding._workspaces[(torch.device(DEV).index, stream, "quantize")][-1]


@pytest.mark.parametrize("rows,cols,fmt", [(8192, 4096, "e5m2"), (4099, 8192, "e4m3fn"),
                                           (8192, 8192, "e4m3fn")])
def test_per_tensor_onepass_shares_left_to_the_last_arrival(rows, cols, fmt):
    # A wait limit of 0: every workgroup of the one-pass kernel but the last
    # to arrive gives up at once and leaves its share to that one, which
    # re-reads it; the codes must not change, and the workspace must be back
    # at zero after the call.
    bits = _workload_bits(rows, cols, key=rows * 5 + cols + len(fmt))
    before = binding.lib().fp8_quantize_set_wait_limit_us(0)
    try:
        check(bits, PT, fmt, True)
    finally:
        binding.lib().fp8_quantize_set_wait_limit_us(before)
    assert not _quantize_ws().view(torch.int32).cpu().numpy().any()


def test_per_tensor_onepass_workspace_is_left_at_zero():
    bits = _workload_bits(8192, 8192, key=77)
    for _ in range(2):
        check(bits, PT, "e4m3fn", True)
        assert not _quantize_ws().view(torch.int32).cpu().numpy().any()


def test_per_tensor_onepass_on_two_streams_at_once():
    # Two calls that may run at the same time, each on its own stream (and so
    # with its own workspace): when they compete for CUs, workgroups that
    # cannot all be resident fall back to the second kernel; the results
    # stay exact.
    xs = [_workload_bits(8192, 8192, key=k) for k in (91, 92)]
    refs = [oracle.quantize(b, PT, oracle.E4M3FN) for b in xs]
    ts = [torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV) for b in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    print("[quantize] two streams, 8192x8192 per-tensor each", flush=True)
    outs = []
    for _ in range(3):
        for t, st in zip(ts, streams):
            with torch.cuda.stream(st):
                outs.append(binding.fp8_quantize(t, PT))
    torch.cuda.synchronize()
    for i, (q, sc) in enumerate(outs):
        rq, rs = refs[i % 2]
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
        assert np.array_equal(q.cpu().numpy(), rq), f"call {i}"


def test_per_tensor_onepass_in_a_graph():
    # Captured once, replayed several times with eager work between the
    # replays: every replay equals the eager result (the workspace's counters
    # are reset by a kernel, never by a memset node).
    bits = _workload_bits(4099, 8192, key=5)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    print("[quantize] graph capture of the per-tensor one-pass path", flush=True)
    q0, s0 = binding.fp8_quantize(x, PT)
    torch.cuda.synchronize()
    ref_q, ref_s = q0.cpu().numpy(), s0.cpu().numpy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q, sc = binding.fp8_quantize(x, PT)          # the workspace of stream s exists before capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            binding.fp8_quantize(x, PT, q=q, scale=sc)
    torch.cuda.synchronize()
    for i in range(3):
        q.zero_()
        sc.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(sc.cpu().numpy(), ref_s), f"replay {i}"
        assert np.array_equal(q.cpu().numpy(), ref_q), f"replay {i}"
        _ = binding.fp8_quantize(x, PT)              # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("rows,cols,fmt", [(40000, 256, "e4m3fn"), (40000, 256, "e5m2"),
                                           (33000, 4112, "e4m3fn")])
def test_rowwise_more_rows_than_workgroups_bitexact(rows, cols, fmt):
    # More rows than the row-wise grid (128 workgroups per CU): workgroups
    # walk several rows with the next row prefetched into registers.
    bits = _workload_bits(rows, cols, key=rows * 3 + cols + len(fmt))
    check(bits, RW, fmt)
