"""Seeded random cases: ragged shapes, both scaling modes, with and without
bias, every operand-format pair, run with a random tile configuration and
split count (or the automatic plan), each compared with the CPU oracle
element by element."""
import numpy as np
import pytest

from precision_linear_amd import binding
from precision_linear_amd import workloads as wl
from parity import compare
from test_gpu_parity import out_bits, ref_mm, run_gpu_plan

pytestmark = pytest.mark.gpu
FORMATS = [("e4m3fn", "e4m3fn"), ("e5m2", "e5m2"), ("e4m3fn", "e5m2"), ("e5m2", "e4m3fn")]
N_CASES = 160


def _case(seed):
    rng = np.random.default_rng([7, seed])
    fa, fb = FORMATS[seed % 4] if seed % 3 else FORMATS[0]
    small = fa != "e4m3fn" or fb != "e4m3fn"      # the exact e5m2 oracle is slower
    M = int(rng.integers(1, 300 if small else 700))
    N = int(rng.integers(1, 300 if small else 700))
    K = 16 * int(rng.integers(1, (1024 if small else 4096) // 16 + 1))
    mode = int(rng.integers(0, 2))
    bias = bool(rng.integers(0, 2))
    n_cfg = len(binding.config_names())
    config = int(rng.integers(-1, n_cfg))          # -1: the automatic choice
    splits = int(rng.choice([0, 1, 2, 3, 5, 8]))
    return M, N, K, mode, bias, fa, fb, config, splits


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_plan(seed):
    M, N, K, mode, bias, fa, fb, config, splits = _case(seed)
    print(f"[random] seed={seed} shape=({M},{N},{K}) mode={mode} bias={bias} {fa}x{fb} "
          f"config={config} splits={splits}", flush=True)
    inp = wl.make_inputs(M, N, K, mode, "codes", bias=bias, key=1000 + seed, a_format=fa,
                         b_format=fb)
    got = out_bits(run_gpu_plan(inp, config, splits))
    nbad, worst, first = compare(got, ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)
