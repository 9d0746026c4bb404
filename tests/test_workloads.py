"""Host-side checks of the seeded input generator (no GPU, no oracle)."""
import numpy as np
import torch

from precision_linear_amd import workloads as wl


def test_deterministic_per_seed():
    x1 = wl.make_inputs(64, 48, 96, wl.ROWWISE, "normal", True, key=123)
    x2 = wl.make_inputs(64, 48, 96, wl.ROWWISE, "normal", True, key=123)
    x3 = wl.make_inputs(64, 48, 96, wl.ROWWISE, "normal", True, key=124)
    assert x1.sha256() == x2.sha256()
    assert x1.sha256()["a"] != x3.sha256()["a"]


def test_amax_quantisation_recipe():
    x = wl.make_inputs(32, 40, 64, wl.ROWWISE, "normal", key=5)
    assert x.a.dtype == np.uint8 and x.a.shape == (32, 64)
    assert x.b.dtype == np.uint8 and x.b.shape == (40, 64)
    assert x.scale_a.shape == (32,) and x.scale_b.shape == (40,)
    # every row reaches the e4m3fn maximum 448 (code 0x7E or 0xFE) at its amax
    for codes in (x.a, x.b):
        assert np.all(np.any((codes & 0x7F) == 0x7E, axis=1))
        assert not np.any((codes & 0x7F) == 0x7F)           # never NaN
    xt = wl.make_inputs(32, 40, 64, wl.PER_TENSOR, "normal", key=5)
    assert xt.scale_a.shape == (1,) and xt.scale_b.shape == (1,)
    assert np.isclose(xt.scale_a[0], np.max(x.scale_a))


def test_codes_recipe():
    x = wl.make_inputs(512, 256, 64, wl.ROWWISE, "codes", key=9)
    assert not np.any((x.a & 0x7F) == 0x7F) and not np.any((x.b & 0x7F) == 0x7F)
    zf = np.mean(x.a == 0)
    assert 0.008 < zf < 0.02                   # 1% planted zeros + 1/254 drawn zeros
    lg = np.log2(x.scale_a.astype(np.float64))
    assert lg.min() >= -8 and lg.max() <= 4


def test_skinny_recipe_has_bias_and_small_weights():
    x = wl.make_inputs(16, 512, 256, wl.ROWWISE, "skinny", True, key=3)
    assert x.bias is not None and x.bias.dtype == np.uint16 and x.bias.shape == (512,)
    bias = torch.from_numpy(x.bias.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert 0.8 < bias.std() < 1.2
    # weights ~ N(0, 0.02): row-wise amax/448 is about 0.02 * 3 / 448
    assert np.median(x.scale_b) < 0.001


def test_workload_table():
    names = list(wl.WORKLOADS)
    assert "sq8192_pt" in names and "sq8192_rw" in names
    assert sum(n.startswith("skinny") for n in names) == 6
    assert sum(n.startswith("ragged") for n in names) == 8
    w = wl.WORKLOADS["sq8192_pt"]
    assert w.flops == 2 * 8192 ** 3
    assert w.algorithmic_bytes == 2 * 8192 * 8192 + 8 + 2 * 8192 * 8192
