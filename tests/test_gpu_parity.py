"""GPU parity: the HIP library against the CPU oracle, element by element,
on seeded inputs, through the C ABI (via the thin ctypes binding).

Small and ragged shapes, and every e4m3fn workload up to M = N = K = 8192,
are compared in full; the largest shape (16384 x 16384 x 8192) and the e5m2
workloads, whose exact integer oracle is slow, on rows and columns that hit
every output tile of the launch.
"""
import re

import numpy as np
import pytest
import torch

import oracle
from precision_linear_amd import binding
from precision_linear_amd import workloads as wl
from parity import bf16_bits_to_f64, compare

pytestmark = pytest.mark.gpu
PT, RW = wl.PER_TENSOR, wl.ROWWISE
DEV = "cuda:0"


def _to_dev(x):
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(DEV)


OFMT = {"e4m3fn": oracle.E4M3FN, "e5m2": oracle.E5M2}


def ref_mm(inp, rows=None, cols=None, bias="inp"):
    """The oracle on an Inputs (its operand formats included)."""
    return oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b,
                            inp.bias if isinstance(bias, str) else bias, inp.mode, rows=rows,
                            cols=cols, a_format=OFMT[inp.a_format], b_format=OFMT[inp.b_format])


def run_gpu(inp, config=-1, out=None):
    a, b = _to_dev(inp.a), _to_dev(inp.b)
    sa, sb = _to_dev(inp.scale_a), _to_dev(inp.scale_b)
    bias = _to_dev(inp.bias)
    out = binding.fp8_scaled_mm(a, b, sa, sb, bias, out=out, mode=inp.mode, config=config,
                                a_format=inp.a_format, b_format=inp.b_format)
    torch.cuda.synchronize()
    return out


def out_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def check_full(inp, config=-1):
    print(f"[parity] shape={inp.shape} mode={inp.mode} bias={inp.bias is not None} "
          f"config={config}", flush=True)
    got = out_bits(run_gpu(inp, config))
    ref = ref_mm(inp)
    nbad, worst, first = compare(got, ref)
    assert nbad == 0, f"{nbad} elements out of bound, worst ratio {worst:.3g}, first {first}"
    return got, ref


def tile_dims(inp, config=-1):
    """(BM, BN) of the tile configuration the call uses (the automatic choice
    for config < 0), read from its name."""
    M, N, K = inp.shape
    cfg = config if config >= 0 else binding.select_config(M, N, K, inp.mode, inp.bias is not None)
    name = binding.config_names()[cfg]
    return int(re.search(r"bm(\d+)", name).group(1)), int(re.search(r"bn(\d+)", name).group(1))


def covering_indices(n, band, rot):
    """One index inside every band of `band` consecutive indices (the last band
    may be short), at an offset that rotates from band to band, plus 0 and n-1.
    With band = the tile's height (width), every tile row (column) of the grid
    contains a chosen index, and the offsets reach different waves and lanes
    of the tiles."""
    idx = [0, n - 1]
    for b in range((n + band - 1) // band):
        lo = b * band
        width = min(band, n - lo)
        idx.append(lo + (b * 37 + rot) % width)
    return np.unique(np.asarray(idx, dtype=np.int64))


def check_sampled(inp, out, config=-1, band_scale=1, rot=0):
    """Compare whole rows and whole columns chosen by covering_indices: one row
    in every tile row and one column in every tile column of the launch's tile
    grid, so every output tile is checked along a full row and a full column.
    band_scale > 1 samples every band_scale-th tile row/column band instead
    (only for the slow e5m2 oracle)."""
    M, N, K = inp.shape
    bm, bn = tile_dims(inp, config)
    rows = covering_indices(M, bm * band_scale, rot)
    cols = covering_indices(N, bn * band_scale, rot + 11)
    print(f"[parity] sampled {len(rows)} rows (band {bm * band_scale}), {len(cols)} cols "
          f"(band {bn * band_scale})", flush=True)
    rows_t = torch.from_numpy(rows).to(out.device)
    cols_t = torch.from_numpy(cols).to(out.device)
    g_rows = out_bits(out.index_select(0, rows_t))
    g_cols = out_bits(out.index_select(1, cols_t))
    r_rows = ref_mm(inp, rows=rows)
    r_cols = ref_mm(inp, cols=cols)
    for g, r, what in ((g_rows, r_rows, "rows"), (g_cols, r_cols, "cols")):
        nbad, worst, first = compare(g, r)
        assert nbad == 0, f"{what}: {nbad} out of bound, worst {worst:.3g}, first {first}"


# ------------------------------------------------------------ small / ragged ---

SMALL_SHAPES = [
    (1, 1, 16), (1, 7, 32), (5, 1, 48), (32, 32, 64), (64, 64, 128),
    (100, 70, 160), (257, 129, 272), (300, 513, 256), (128, 96, 4096 + 48),
    (513, 260, 96), (33, 1000, 528),
]


@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_shapes_auto_config(shape, mode):
    M, N, K = shape
    inp = wl.make_inputs(M, N, K, mode, "codes", bias=(M + N) % 2 == 0, key=M * 7 + N * 13 + K)
    check_full(inp)


def _configs():
    return list(range(len(binding.config_names())))


def _config_ids():
    return [f"{i}_{n}" for i, n in enumerate(binding.config_names())]


@pytest.mark.parametrize("config", _configs(), ids=_config_ids())
@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("shape", [(300, 200, 160), (257, 515, 400), (64, 128, 1024), (16, 300, 2080)])
def test_every_config_ragged(config, mode, bias, shape):
    M, N, K = shape
    inp = wl.make_inputs(M, N, K, mode, "codes", bias=bias, key=config * 101 + M + N + K)
    check_full(inp, config)


@pytest.mark.parametrize("config", _configs(), ids=_config_ids())
@pytest.mark.parametrize("shape", [(200, 1026, 256), (140, 766, 128), (129, 4097, 32)])
def test_every_config_unaligned_rows(config, shape):
    # Rows that do not start on a 16-byte boundary (N % 8 = 2, 6 and odd):
    # every row start phase N allows (2 bytes apart for odd N), heads of 0-7
    # values, tails, and tiles narrower than 8 columns at the right edge.
    M, N, K = shape
    inp = wl.make_inputs(M, N, K, RW, "codes", bias=True, key=config * 31 + N)
    check_full(inp, config)


@pytest.mark.parametrize("recipe", ["normal", "skinny"])
def test_normal_inputs_small(recipe):
    inp = wl.make_inputs(192, 320, 512, RW, recipe, bias=recipe == "skinny", key=77)
    check_full(inp)


# ------------------------------------------------------- bitwise invariants ---

def _small(mode=PT, bias=False, key=5, shape=(130, 200, 288)):
    return wl.make_inputs(*shape, mode, "codes", bias=bias, key=key)


def test_deterministic():
    inp = _small(RW, True)
    a = out_bits(run_gpu(inp))
    b = out_bits(run_gpu(inp))
    assert np.array_equal(a, b)


def test_power_of_two_scale_is_exact():
    inp = _small(PT)
    base = bf16_bits_to_f64(out_bits(run_gpu(inp)))
    inp.scale_a = (inp.scale_a * np.float32(8.0)).astype(np.float32)
    scaled = bf16_bits_to_f64(out_bits(run_gpu(inp)))
    ok = np.abs(base) > 2.0 ** -120
    assert np.array_equal(scaled[ok], 8.0 * base[ok])


def test_rowwise_constant_equals_per_tensor_bitwise():
    inp = _small(PT, True)
    pt = out_bits(run_gpu(inp))
    M, N, _ = inp.shape
    inp_rw = wl.Inputs(inp.a, inp.b, np.repeat(inp.scale_a, M), np.repeat(inp.scale_b, N),
                       inp.bias, RW)
    rw = out_bits(run_gpu(inp_rw))
    assert np.array_equal(pt, rw)


def test_sign_flip_negates_bitwise():
    inp = _small(RW)
    a = out_bits(run_gpu(inp))
    inp_neg = wl.Inputs(inp.a ^ np.uint8(0x80), inp.b, inp.scale_a, inp.scale_b, None, RW)
    b = out_bits(run_gpu(inp_neg))
    nz = (a & 0x7FFF) != 0
    assert np.array_equal(b[nz], a[nz] ^ np.uint16(0x8000))


def test_zero_k_padding_bitwise():
    inp = _small(RW, True, shape=(96, 80, 96))
    a = out_bits(run_gpu(inp))
    M, N, K = inp.shape
    pad = 160
    inp_p = wl.Inputs(np.concatenate([inp.a, np.zeros((M, pad), np.uint8)], 1),
                      np.concatenate([inp.b, np.zeros((N, pad), np.uint8)], 1),
                      inp.scale_a, inp.scale_b, inp.bias, RW)
    b = out_bits(run_gpu(inp_p))
    assert np.array_equal(a, b)


def test_identity_is_exact():
    K = 256
    a = np.zeros((K, K), np.uint8)
    a[np.arange(K), np.arange(K)] = 0x38
    bsrc = _small(PT, shape=(8, 200, K))
    inp = wl.Inputs(a, bsrc.b, np.array([0.5], np.float32), np.array([4.0], np.float32), None, PT)
    got = out_bits(run_gpu(inp))
    dec = torch.from_numpy(bsrc.b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    want = oracle.f64_to_bf16_rne(2.0 * dec.T)
    want = np.where(want == 0x8000, np.uint16(0), want)
    got = np.where(got == 0x8000, np.uint16(0), got)
    assert np.array_equal(got, want)


def _rounding_inputs(M, N, K, mode, key):
    """One-hot rows of A (code 0x38 = 1.0 at column m % K) make every fp32
    accumulator one e4m3 value of B exactly; scale_b = 1 makes s = scale_a
    exactly; an e4m3 value (at most 4 significant bits) times a scale of at most
    20 significant bits is exact in fp32.  The conversion to bf16 is then the
    only rounding, so the output must match the oracle bit for bit.  The row
    scales include exact bf16 ties (1 + k*2^-7 + 2^-8, which round to even),
    20-bit values, and values near 2^-128 whose products land in the bf16
    denormal range."""
    rng = np.random.Generator(np.random.PCG64(key))
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), np.arange(M) % K] = 0x38
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    b = codes[rng.integers(0, len(codes), (N, K))]
    n = M if mode == RW else 1
    kind = rng.integers(0, 3, n)
    tie = (1.0 + rng.integers(0, 128, n) * 2.0 ** -7 + 2.0 ** -8) * 2.0 ** rng.integers(-20, 21, n)
    wide = (1.0 + rng.integers(0, 2 ** 19, n) * 2.0 ** -19) * 2.0 ** rng.integers(-20, 21, n)
    tiny = (1.0 + rng.integers(0, 16, n) / 16.0) * 2.0 ** -128
    sa = np.where(kind == 0, tie, np.where(kind == 1, wide, tiny))
    sa = (sa * np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0)).astype(np.float32)
    assert np.array_equal(sa.astype(np.float64), np.where(kind == 0, tie, np.where(kind == 1, wide, tiny))
                          * np.sign(sa.astype(np.float64)))
    sb = np.ones(N if mode == RW else 1, np.float32)
    return wl.Inputs(a, b, sa, sb, None, mode)


@pytest.mark.parametrize("config", _configs(), ids=_config_ids())
@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("shape", [(512, 256, 64), (300, 200, 64)])
def test_epilogue_rounding_bitexact(config, mode, shape):
    inp = _rounding_inputs(*shape, mode, key=config * 7 + mode + shape[0])
    got = out_bits(run_gpu(inp, config))
    want = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, None, mode)["bits"]
    # +0 and -0 are the same value (the fp32 accumulator of a zero product sum
    # is +0 on the GPU, and the sign of s then decides the sign of zero)
    got = np.where(got == 0x8000, np.uint16(0), got)
    want = np.where(want == 0x8000, np.uint16(0), want)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"got {got[tuple(bad[0])]:#06x} want {want[tuple(bad[0])]:#06x}")


def test_every_element_written():
    inp = _small(RW, True, shape=(259, 131, 64))
    M, N, _ = inp.shape
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    run_gpu(inp, out=out)
    assert not torch.isnan(out).any()


def test_empty_is_noop():
    inp = _small(PT, shape=(16, 16, 32))
    a, b = _to_dev(inp.a), _to_dev(inp.b)
    sa, sb = _to_dev(inp.scale_a), _to_dev(inp.scale_b)
    out = torch.full((0, 16), 1.0, dtype=torch.bfloat16, device=DEV)
    binding.fp8_scaled_mm(a[:0], b, sa, sb, out=out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("offset,N", [(1, 131), (4, 136)])
def test_unaligned_output_rows_fall_back(offset, N):
    """An output base that is only 2- (or 8-) byte aligned: the kernel must not
    use its 16-byte stores on rows that do not start on a 16-byte boundary,
    even where N % 8 == 0."""
    inp = _small(RW, True, shape=(70, N, 128))
    M = inp.shape[0]
    buf = torch.full((M * N + offset,), float("nan"), dtype=torch.bfloat16, device=DEV)
    out = buf[offset:].view(M, N)
    run_gpu(inp, out=out)
    ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias, RW)
    nbad, worst, first = compare(out_bits(out), ref)
    assert nbad == 0, (nbad, worst, first)


def test_column_major_b_view():
    inp = _small(PT, shape=(64, 96, 128))
    a, b = _to_dev(inp.a), _to_dev(inp.b)
    b_kn = b.t()                                   # K x N, stride (1, K)
    sa, sb = _to_dev(inp.scale_a), _to_dev(inp.scale_b)
    o1 = binding.fp8_scaled_mm(a, b, sa, sb)
    o2 = binding.fp8_scaled_mm(a, b_kn, sa, sb)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ------------------------------------------- full-size workloads (sampled) ---

@pytest.mark.parametrize("name", [n for n in wl.WORKLOADS if not n.startswith("ragged_16384")])
def test_workload(name):
    inp = wl.make_workload(name)
    print(f"[parity] workload {name} shape={inp.shape}", flush=True)
    out = run_gpu(inp)
    M, N, K = inp.shape
    e4m3 = inp.a_format == inp.b_format == "e4m3fn"
    if e4m3 or M * N * K <= 1024 ** 3:
        # every output element, up to the M = N = K = 8192 headline shape
        ref = ref_mm(inp)
        nbad, worst, first = compare(out_bits(out), ref)
        print(f"[parity] full compare: worst error {worst:.3f} of the bound", flush=True)
        assert nbad == 0, (nbad, worst, first)
    else:
        # e5m2: the oracle's exact integer sums are slow; one row in every
        # tile row and one column in every tile column
        check_sampled(inp, out, rot=len(name))


@pytest.mark.slow
@pytest.mark.parametrize("name", [n for n in wl.WORKLOADS if n.startswith("ragged_16384")])
def test_workload_largest(name):
    inp = wl.make_workload(name)
    print(f"[parity] workload {name} shape={inp.shape}", flush=True)
    out = run_gpu(inp)
    check_sampled(inp, out, rot=len(name))


# ------------------------------------ ping-pong kernel: several tiles per CU ---

@pytest.mark.parametrize("shape", [(4352, 4096, 512), (8192, 8192, 128), (8192, 8192, 256),
                                   (4400, 4104, 384), (6144, 6144, 2176)])
@pytest.mark.parametrize("mode,bias", [(PT, False), (RW, True), (PT, True)])
def test_ping_pong_several_tiles_per_workgroup(shape, mode, bias):
    # More 256 x 256 tiles than workgroups (272, 1024, 1024, 306, 576 tiles on
    # 256 CUs): workgroups change tiles, so the tile-change path (outputs of
    # one tile, then the next tile's first slices and epilogue parameters,
    # alternating parameter areas) runs; units of 1, 2, 3, 4 and 17 slices;
    # ragged edge tiles in (4400, 4104, 384).  Compared in full.
    M, N, K = shape
    pp = _cfg("pp_bm256_bn256_bk128_w8_mfma16")
    inp = wl.make_inputs(M, N, K, mode, "codes", bias=bias, key=M + N + K + 3 * mode + bias)
    print(f"[parity] ping-pong shape={shape} mode={mode} bias={bias}", flush=True)
    got = out_bits(run_gpu_plan(inp, pp, 1))
    nbad, worst, first = compare(got, ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)


@pytest.mark.parametrize("mode", [PT, RW])
def test_ping_pong_several_units_per_workgroup_split(mode):
    # split-K units: 272 tiles x 2 splits = 544 units on 256 workgroups
    M, N, K = 4352, 4096, 10240
    pp = _cfg("pp_bm256_bn256_bk128_w8_mfma16")
    inp = wl.make_inputs(M, N, K, mode, "codes", bias=mode == RW, key=90 + mode)
    got = out_bits(run_gpu_plan(inp, pp, 2))
    nbad, worst, first = compare(got, ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)


# ---------------------------------------------------------------- split-K ---

def _cfg(name):
    return binding.config_names().index(name)


@pytest.mark.parametrize("config", ["bm128_bn128_bk128_w2x2_s2_mfma32", "bm16_bn64_bk256_w1x4_s4_mfma16",
                                    "bm16_bn112_bk256_w1x7_s4_mfma16", "bm64_bn112_bk256_w1x7_s3_mfma16",
                                    "bm64_bn64_bk256_w1x4_s4_mfma16", "bm128_bn128_bk128_w2x4_s4_mfma32",
                                    "pp_bm256_bn256_bk128_w8_mfma16", "bm128_bn32_bk256_w4x2_s3_mfma16",
                                    "bm64_bn32_bk256_w4x2_s4_mfma16", "bm128_bn64_bk256_w4x2_s3_mfma16",
                                    "bm16_bn32_bk512_w1x2_s6_mfma16"])
@pytest.mark.parametrize("splits", [2, 3, 4, 7])
@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("M", [150, 16])
def test_split_k_parity(config, splits, mode, M):
    # K = 1040: 9 slices of 128 (last ragged), so splits do not divide it evenly.
    # M = 16 gives a single row of tiles (the non-temporal-B launch).
    inp = wl.make_inputs(M, 230, 1040, mode, "codes", bias=mode == RW, key=splits * 7 + mode + M)
    got = out_bits(run_gpu_plan(inp, _cfg(config), splits))
    ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias, inp.mode)
    nbad, worst, first = compare(got, ref)
    assert nbad == 0, (nbad, worst, first)


@pytest.mark.parametrize("splits", [2, 3])
@pytest.mark.parametrize("mode", [PT, RW])
def test_split_k_ping_pong_full_tiles(splits, mode):
    # whole 256 x 256 tiles (16-byte staged stores) plus a ragged edge tile,
    # K = 4160: 33 slices, so the units have 17 + 16 or 11 + 11 + 11 slices
    inp = wl.make_inputs(520, 768, 4160, mode, "codes", bias=mode == RW, key=40 + splits + mode)
    pp = _cfg("pp_bm256_bn256_bk128_w8_mfma16")
    got = out_bits(run_gpu_plan(inp, pp, splits))
    nbad, worst, first = compare(got, ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)
    ws = torch.zeros(binding.workspace_size(520, 768, 4160, mode, mode == RW, pp, splits),
                     dtype=torch.uint8, device=DEV)
    again = out_bits(run_gpu_plan(inp, pp, splits, workspace=ws))
    assert np.array_equal(got, again)          # deterministic whatever the arrival order
    assert int(ws[:262144].sum()) == 0         # every (tile, wave) counter back at zero


def run_gpu_plan(inp, config, splits, workspace=None, out=None):
    a, b = _to_dev(inp.a), _to_dev(inp.b)
    sa, sb = _to_dev(inp.scale_a), _to_dev(inp.scale_b)
    bias = _to_dev(inp.bias)
    out = binding.fp8_scaled_mm(a, b, sa, sb, bias, out=out, mode=inp.mode, config=config,
                                splits=splits, workspace=workspace, a_format=inp.a_format,
                                b_format=inp.b_format)
    torch.cuda.synchronize()
    return out


def test_split_k_more_splits_than_slices():
    inp = wl.make_inputs(64, 96, 256, PT, "codes", key=3)
    got = out_bits(run_gpu_plan(inp, _cfg("bm128_bn128_bk128_w2x2_s2_mfma32"), 16))
    ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, None, PT)
    assert compare(got, ref)[0] == 0


@pytest.mark.parametrize("config,splits", [("bm16_bn32_bk512_w1x2_s6_mfma16", 32),
                                           ("bm16_bn64_bk256_w1x4_s4_mfma16", 24),
                                           ("bm64_bn32_bk256_w4x2_s4_mfma16", 16),
                                           ("bm128_bn128_bk128_w2x4_s4_mfma32", 32),
                                           ("bm128_bn128_bk128_w2x2_s2_mfma32", 24)])
@pytest.mark.parametrize("mode", [PT, RW])
def test_split_k_many_splits(config, splits, mode):
    # The automatic plan splits up to 32 ways: K = 16400 (33 slices of 512,
    # 65 of 256, 129 of 128, the last one ragged), so units have 1-6 slices
    # and the last unit of a tile sums up to 32 partials in split order.
    inp = wl.make_inputs(40, 200, 16400, mode, "codes", bias=mode == RW, key=splits + 5 * mode)
    got = out_bits(run_gpu_plan(inp, _cfg(config), splits))
    nbad, worst, first = compare(got, ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)


def test_split_k_deterministic_and_workspace_equivalent():
    inp = wl.make_inputs(128, 512, 8192, RW, "normal", bias=True, key=11)
    cfg = _cfg("bm128_bn128_bk128_w2x2_s2_mfma32")
    r1 = out_bits(run_gpu_plan(inp, cfg, 8))
    r2 = out_bits(run_gpu_plan(inp, cfg, 8))
    need = binding.workspace_size(128, 512, 8192, RW, True, cfg, 8)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    r3 = out_bits(run_gpu_plan(inp, cfg, 8, workspace=ws))
    r4 = out_bits(run_gpu_plan(inp, cfg, 8, workspace=ws))      # left zero-filled by r3
    assert np.array_equal(r1, r2) and np.array_equal(r1, r3) and np.array_equal(r1, r4)
    assert int(ws[:262144].sum()) == 0                            # counters back at zero
    ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias, RW)
    assert compare(r1, ref)[0] == 0


def test_split_k_changing_plans_on_one_stream():
    cfg = _cfg("bm128_bn128_bk128_w2x2_s2_mfma32")
    # the 1-tile plan leaves non-zero partials right after the counters of a
    # small plan; the 72-tile plan that follows must still find zero counters
    for i, (shape, splits) in enumerate([((256, 384, 2048), 4), ((128, 256, 4096), 2),
                                         ((256, 384, 2048), 8), ((300, 130, 1552), 3),
                                         ((128, 128, 8192), 8), ((1024, 1152, 2048), 2)]):
        inp = wl.make_inputs(*shape, PT, "codes", key=100 + i)
        got = out_bits(run_gpu_plan(inp, cfg, splits))
        ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, None, PT)
        assert compare(got, ref)[0] == 0, (shape, splits)


# ------------------------------------------------------------------ stream-K ---

def _sk_configs():
    # every configuration with a stream-K form (split-K capable, not ping-pong)
    L = binding.lib()
    return [c for c, n in enumerate(binding.config_names())
            if L.fp8_scaled_mm_workspace_size(512, 512, 4096, 1, 0, c, binding.SPLITS_STREAM_K) > 0]


@pytest.mark.parametrize("config", _sk_configs(),
                         ids=[binding.config_names()[c] for c in _sk_configs()])
@pytest.mark.parametrize("shape,mode,bias", [((300, 200, 1040), PT, True),
                                             ((640, 768, 4096), RW, True),
                                             ((1000, 1200, 2048), RW, False)])
def test_stream_k_parity(config, shape, mode, bias):
    # 6, 30 and 80 tiles of 128 x 128 over every workgroup slot of the GPU: each
    # tile shared by several workgroups (one K slice each for the first shape),
    # ranges that end inside tiles and start inside the next, ragged edges
    inp = wl.make_inputs(*shape, mode, "codes", bias=bias, key=config * 7 + shape[0])
    got = out_bits(run_gpu_plan(inp, config, binding.SPLITS_STREAM_K))
    ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias, mode)
    nbad, worst, first = compare(got, ref)
    assert nbad == 0, (nbad, worst, first)


def test_stream_k_deterministic_and_counters_left_zero():
    inp = wl.make_inputs(512, 3072, 4096, RW, "normal", bias=True, key=13)
    cfg = _cfg("bm128_bn128_bk128_w2x2_s2_mfma32")
    need = binding.workspace_size(512, 3072, 4096, RW, True, cfg, binding.SPLITS_STREAM_K)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    r1 = out_bits(run_gpu_plan(inp, cfg, binding.SPLITS_STREAM_K, workspace=ws))
    r2 = out_bits(run_gpu_plan(inp, cfg, binding.SPLITS_STREAM_K, workspace=ws))
    r3 = out_bits(run_gpu_plan(inp, cfg, binding.SPLITS_STREAM_K))
    assert np.array_equal(r1, r2) and np.array_equal(r1, r3)
    assert int(ws[:262144].sum()) == 0                            # counters back at zero
    ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias, RW)
    assert compare(r1, ref)[0] == 0


def test_tensors_on_another_device_are_refused():
    # every pointer goes to a kernel on the operands' GPU: a host tensor
    # anywhere in the call must be refused before anything is launched
    inp = wl.make_inputs(64, 96, 128, RW, "codes", bias=True, key=5)
    a, b = _to_dev(inp.a), _to_dev(inp.b)
    sa, sb, bias = _to_dev(inp.scale_a), _to_dev(inp.scale_b), _to_dev(inp.bias)
    cpu_out = torch.empty(64, 96, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, b, sa, sb, bias, out=cpu_out, mode=RW)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, b, sa, sb, bias.cpu(), mode=RW)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, b, sa, sb, bias, mode=RW, splits=2,
                              workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, b, sa.cpu(), sb, bias, mode=RW)
    out = binding.fp8_scaled_mm(a, b, sa, sb, bias, mode=RW)    # and the good call still works
    torch.cuda.synchronize()
    nbad, worst, first = compare(out_bits(out), ref_mm(inp))
    assert nbad == 0


def test_split_k_on_two_streams_at_once():
    # calls on different streams use different library workspaces: split-K
    # multiplies of different shapes, queued on two streams without any
    # synchronisation between them, both match the oracle
    inps = [wl.make_inputs(128, 1024, 4096, RW, "skinny", bias=True, key=61),
            wl.make_inputs(64, 2048, 6144, PT, "skinny", bias=False, key=62)]
    args = [[_to_dev(x) for x in (i.a, i.b, i.scale_a, i.scale_b, i.bias)] for i in inps]
    for i in inps:
        assert binding.select_splits(*i.shape, i.mode, i.bias is not None) > 1
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty(i.shape[0], i.shape[1], dtype=torch.bfloat16, device="cuda")
            for i in inps]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for k in (0, 1):
            with torch.cuda.stream(streams[k]):
                for _ in range(4):
                    binding.fp8_scaled_mm(*args[k][:4], args[k][4], out=outs[k], mode=inps[k].mode)
    torch.cuda.synchronize()
    for k in (0, 1):
        nbad, worst, first = compare(out_bits(outs[k]), ref_mm(inps[k]))
        assert nbad == 0, (k, nbad, worst, first)


@pytest.mark.parametrize("config,splits", [(-1, 0), ("pp_bm256_bn256_bk128_w8_mfma16", 1),
                                           ("bm128_bn128_bk128_w2x4_s4_mfma32", 1),
                                           ("bm16_bn112_bk256_w1x7_s4_mfma16", 1),
                                           ("bm128_bn128_bk128_w2x4_s4_mfma32", 3),
                                           ("bm128_bn128_bk128_w2x2_s2_mfma32", 2)])
@pytest.mark.parametrize("mode", [PT, RW])
def test_nan_codes_propagate(config, splits, mode):
    # e4m3fn NaN codes (0x7F, 0xFF) in A and B: every output whose dot
    # product meets one is NaN (the oracle's fp64 sum propagates it), every
    # other output is unchanged; the comparison demands NaN where the
    # reference is NaN
    inp = wl.make_inputs(300, 520, 640, mode, "codes", bias=mode == RW, key=71 + mode)
    a, b = inp.a.copy(), inp.b.copy()
    a[5, 17] = 0x7F
    a[211, 600] = 0xFF
    b[33, 0] = 0x7F
    b[519, 639] = 0xFF
    inp = wl.Inputs(a, b, inp.scale_a, inp.scale_b, inp.bias, mode, "e4m3fn", "e4m3fn")
    got = out_bits(run_gpu_plan(inp, config if config == -1 else _cfg(config), splits))
    ref = ref_mm(inp)
    nbad, worst, first = compare(got, ref)
    assert nbad == 0, (nbad, worst, first)
    vals = bf16_bits_to_f64(got)
    assert np.isnan(vals[5]).all() and np.isnan(vals[211]).all()
    assert np.isnan(vals[:, 33]).all() and np.isnan(vals[:, 519]).all()
    assert np.isfinite(np.delete(np.delete(vals, [5, 211], 0), [33, 519], 1)).all()


@pytest.mark.parametrize("config", _configs(), ids=_config_ids())
@pytest.mark.parametrize("N", [375, 257, 519, 8])
@pytest.mark.parametrize("mode", [PT, RW])
def test_zero_a_gives_the_bias_in_every_column(config, N, mode):
    # A = 0: every output is exactly bf16(bias[n]) (the fp32 accumulator is 0,
    # so fma(0, s, bias) = bias).  Odd and even numbers of columns in the last
    # column tile, and a bias that is only 2-byte aligned: no bias value may
    # be lost or shifted.  (A 16-byte LDS-direct load of the bias whose record
    # limit ended inside a dword once read the last bias value as 0.)
    M, K = 300, 128
    inp = wl.make_inputs(M, N, K, mode, "codes", bias=True, key=N + 7 * mode + 13 * config)
    a = torch.zeros((M, K), dtype=torch.uint8, device=DEV)
    b, sa, sb = _to_dev(inp.b), _to_dev(inp.scale_a), _to_dev(inp.scale_b)
    buf = torch.empty(N + 1, dtype=torch.bfloat16, device=DEV)
    bias = buf[1:]                                          # 2-byte aligned, not 4
    bias.copy_(_to_dev(inp.bias))
    assert bias.data_ptr() % 4 == 2
    out = binding.fp8_scaled_mm(a, b, sa, sb, bias, mode=mode, config=config)
    torch.cuda.synchronize()
    got = out_bits(out)
    want = np.broadcast_to(inp.bias, (M, N))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ from the bias, first at {tuple(bad[0])}"
