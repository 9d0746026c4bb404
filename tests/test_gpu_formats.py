"""GPU parity of the e5m2 and mixed-format multiplies (fp8_scaled_mm_typed,
through the C ABI via the ctypes binding) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from precision_linear_amd import binding
from precision_linear_amd import workloads as wl
from parity import compare
from test_gpu_parity import (OFMT, _cfg, _config_ids, _configs, _to_dev, out_bits, ref_mm, run_gpu,
                             run_gpu_plan)

pytestmark = pytest.mark.gpu
PT, RW = wl.PER_TENSOR, wl.ROWWISE
DEV = "cuda:0"
PAIRS = [("e5m2", "e5m2"), ("e4m3fn", "e5m2"), ("e5m2", "e4m3fn")]
PAIR_IDS = [f"{a}x{b}" for a, b in PAIRS]


def _inputs(M, N, K, mode, fa, fb, recipe="codes", bias=False, key=0):
    return wl.make_inputs(M, N, K, mode, recipe, bias=bias, key=key, a_format=fa, b_format=fb)


def _check(inp, config=-1):
    print(f"[formats] shape={inp.shape} {inp.a_format}x{inp.b_format} mode={inp.mode} "
          f"bias={inp.bias is not None} config={config}", flush=True)
    got = out_bits(run_gpu(inp, config))
    nbad, worst, first = compare(got, ref_mm(inp))
    assert nbad == 0, f"{nbad} out of bound, worst ratio {worst:.3g}, first {first}"
    return got


# Every configuration, every mixed/e5m2 pair: a ragged shape that spans
# several tiles of every config, and a single-row-of-tiles shape (M = 16,
# the non-temporal-B launch of the configs that have one).
@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("config", _configs(), ids=_config_ids())
@pytest.mark.parametrize("shape", [(150, 270, 544), (16, 300, 1040)])
def test_every_config(pair, config, shape):
    M, N, K = shape
    mode = RW if M == 16 else PT
    _check(_inputs(M, N, K, mode, *pair, bias=mode == RW, key=config + 31 * M), config)


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("mode", [PT, RW])
@pytest.mark.parametrize("shape", [(1, 1, 16), (33, 65, 48), (257, 129, 272), (513, 260, 96)])
def test_small_shapes_auto_config(pair, mode, shape):
    _check(_inputs(*shape, mode, *pair, key=sum(shape)))


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("mode", [PT, RW])
def test_normal_recipe(pair, mode):
    # the gist's quantisation of N(0,1) data for each operand's format
    _check(_inputs(200, 300, 1024, mode, *pair, recipe="normal", key=3 + mode))


@pytest.mark.parametrize("config", [0, 8, 11])    # 16 x 32, 128 x 128, ping-pong
def test_recoded_e4m3_values_give_identical_bits(config):
    """e4m3fn values that e5m2 holds exactly (mantissa low bit 0), re-coded
    as e5m2: same products, so the output must not change by a bit."""
    inp = _inputs(300, 260, 512, RW, "e4m3fn", "e4m3fn", key=7)
    a = inp.a & np.uint8(0xFE)                         # clear the lowest mantissa bit
    a[(a & 0x78) == 0] = 0                            # and drop e4m3 subnormals (not all fit)
    b = inp.b & np.uint8(0xFE)
    b[(b & 0x78) == 0] = 0
    a5 = oracle.encode_rne(oracle.decode(a), oracle.E5M2)
    b5 = oracle.encode_rne(oracle.decode(b), oracle.E5M2)
    assert np.array_equal(oracle.decode(a5, oracle.E5M2), oracle.decode(a))
    dev = [_to_dev(x) for x in (a, b, a5, b5, inp.scale_a, inp.scale_b)]
    outs = []
    for (x, y, fa, fb) in ((dev[0], dev[1], "e4m3fn", "e4m3fn"), (dev[2], dev[3], "e5m2", "e5m2"),
                           (dev[0], dev[3], "e4m3fn", "e5m2"), (dev[2], dev[1], "e5m2", "e4m3fn")):
        outs.append(out_bits(binding.fp8_scaled_mm(x, y, dev[4], dev[5], mode=RW, config=config,
                                                   a_format=fa, b_format=fb)))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("config", [0, 1, 8, 9, 10, 11])   # ids: see binding.config_names()
def test_epilogue_rounding_bitexact(pair, config):
    """One-hot A (code 1.0 at column m): out[m, n] = RNE(s * b[n, m]) exactly,
    whatever the format of each operand."""
    fa, fb = pair
    M, N, K = 64, 200, 64
    rng = np.random.default_rng(config)
    one = 0x3C if fa == "e5m2" else 0x38
    a = np.zeros((M, K), np.uint8)
    a[np.arange(M), np.arange(M)] = one
    pool = wl._FINITE_CODES[fb]
    b = pool[rng.integers(0, pool.size, (N, K))]
    sa = np.exp2(rng.uniform(-6, 6, M)).astype(np.float32)
    sb = np.exp2(rng.uniform(-6, 6, N)).astype(np.float32)
    inp = wl.Inputs(a, b, sa, sb, None, RW, fa, fb)
    got = out_bits(run_gpu(inp, config))
    assert np.array_equal(got, ref_mm(inp)["bits"])


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("config,splits", [(9, 3), (1, 4), (6, 2), (10, 2)])
def test_split_k(pair, config, splits):
    inp = _inputs(150, 230, 1040, RW, *pair, bias=True, key=splits)
    a, b = _to_dev(inp.a), _to_dev(inp.b)
    sa, sb, bias = _to_dev(inp.scale_a), _to_dev(inp.scale_b), _to_dev(inp.bias)
    out = binding.fp8_scaled_mm(a, b, sa, sb, bias, mode=RW, config=config, splits=splits,
                                a_format=pair[0], b_format=pair[1])
    torch.cuda.synchronize()
    nbad, worst, first = compare(out_bits(out), ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)


def test_torch_float8_dtypes_carry_the_format():
    inp = _inputs(64, 96, 128, PT, "e5m2", "e4m3fn", key=9)
    a = _to_dev(inp.a).view(torch.float8_e5m2)
    b = _to_dev(inp.b).view(torch.float8_e4m3fn)
    out = binding.fp8_scaled_mm(a, b, _to_dev(inp.scale_a), _to_dev(inp.scale_b))
    torch.cuda.synchronize()
    nbad, worst, first = compare(out_bits(out), ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, b, _to_dev(inp.scale_a), _to_dev(inp.scale_b), a_format="e4m3fn")


# e5m2 infinities and NaNs in the operands (+inf 0x7C, -inf 0xFC, NaN 0x7E,
# 0x7F): the oracle applies IEEE 754 (inf * 0 = NaN, inf - inf = NaN, a lone
# infinity keeps its sign); the comparison demands the same NaN positions and
# the same infinities.  A row of A with one +inf (its outputs are +-inf, or
# NaN where B has a zero at that k), a row with +inf and -inf (NaN), a NaN
# row; in B a -inf column and a NaN column.  The "codes" recipe draws 1% zero
# codes, so inf * 0 occurs too.  Plans: the main tile families and split-K.
NONFINITE_PLANS = [("bm16_bn64_bk256_w1x4_s4_mfma16", 1), ("bm128_bn128_bk128_w2x4_s4_mfma32", 1),
                   ("bm128_bn128_bk128_w2x2_s2_mfma32", 1), ("bm64_bn128_bk128_w2x2_s2_mfma32", 1),
                   ("pp_bm256_bn256_bk128_w8_mfma16", 1), ("bm128_bn128_bk128_w2x4_s4_mfma32", 3),
                   ("pp_bm256_bn256_bk128_w8_mfma16", 2)]


@pytest.mark.parametrize("pair", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("config,splits", NONFINITE_PLANS)
def test_nonfinite_e5m2_codes_follow_ieee(pair, config, splits):
    fa, fb = pair
    inp = _inputs(300, 520, 1024, RW, fa, fb, bias=True, key=splits * 7 + len(config))
    a, b = inp.a.copy(), inp.b.copy()
    if fa == "e5m2":
        a[5, 17] = 0x7C
        a[40, 3], a[40, 9] = 0x7C, 0xFC
        a[77, 100] = 0x7E
    if fb == "e5m2":
        b[33, 0] = 0xFC
        b[200, 5] = 0x7F
    inp = wl.Inputs(a, b, inp.scale_a, inp.scale_b, inp.bias, RW, fa, fb)
    print(f"[formats] non-finite {fa}x{fb} config={config} splits={splits}", flush=True)
    got = out_bits(run_gpu_plan(inp, _cfg(config), splits))
    ref = ref_mm(inp)
    nbad, worst, first = compare(got, ref)
    assert nbad == 0, (nbad, worst, first)
    r = ref["bits"]
    assert (r == 0x7FC0).any() and ((r & 0x7FFF) == 0x7F80).any()    # both kinds occur
