"""fp8_scaled_mm_noalloc -- the entry point for callers that cannot allocate
-- against fp8_scaled_mm_with_plan (the same tile configuration and split
count, with a caller workspace), through the C ABI: two calls in a row on the
same GPU (so the second finds the scratch as the first left it), the second
with a smaller problem; both bit-identical to the workspace form and within
the oracle's tolerance."""
import ctypes

import numpy as np
import pytest
import torch

from precision_linear_amd import binding
from precision_linear_amd import workloads as wl
from parity import compare
from test_gpu_parity import _to_dev, out_bits, ref_mm

pytestmark = pytest.mark.gpu
PT, RW = wl.PER_TENSOR, wl.ROWWISE


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _args(inp):
    return [_to_dev(x) for x in (inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias)]


def _noalloc(L, args, out, inp, config, splits):
    a, b, sa, sb, bias = args
    M, N, K = inp.shape
    return L.fp8_scaled_mm_noalloc(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), _ptr(bias), _ptr(out),
                                   M, N, K, inp.mode,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                   config, splits)


def _with_plan(L, args, out, inp, config, splits):
    a, b, sa, sb, bias = args
    M, N, K = inp.shape
    need = L.fp8_scaled_mm_workspace_size(M, N, K, inp.mode, int(bias is not None), config, splits)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    st = L.fp8_scaled_mm_with_plan(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), _ptr(bias), _ptr(out),
                                   M, N, K, inp.mode,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream),
                                   config, splits, _ptr(ws), ws.numel())
    return st, ws


CASES = [
    # (first, second): the second call is smaller than the first
    (((128, 8192, 28672, RW, True, "skinny"), -1, 0), ((64, 2048, 8192, RW, True, "skinny"), -1, 0)),
    (((520, 768, 4160, PT, False, "codes"), "pp_bm256_bn256_bk128_w8_mfma16", 3),
     ((300, 260, 1040, RW, True, "codes"), "pp_bm256_bn256_bk128_w8_mfma16", 2)),
    (((150, 230, 1040, RW, True, "codes"), "bm128_bn32_bk256_w4x2_s3_mfma16", 4),
     ((16, 200, 1040, PT, False, "codes"), "bm16_bn32_bk512_w1x2_s6_mfma16", 2)),
    # stream-K plans (splits -1)
    (((640, 768, 4096, RW, True, "codes"), "bm128_bn128_bk128_w2x2_s2_mfma32", -1),
     ((300, 200, 1040, PT, False, "codes"), "bm128_bn128_bk128_w2x4_s4_mfma32", -1)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_the_workspace_form(case):
    L = binding.lib()
    names = binding.config_names()
    for k, ((M, N, K, mode, bias, recipe), config, splits) in enumerate(CASES[case]):
        cfg = names.index(config) if isinstance(config, str) else config
        inp = wl.make_inputs(M, N, K, mode, recipe, bias=bias, key=500 + 10 * case + k)
        print(f"[noalloc] case {case} call {k}: shape={inp.shape} mode={mode} bias={bias} "
              f"config={cfg} splits={splits}", flush=True)
        args = _args(inp)
        out_n = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        out_w = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert _noalloc(L, args, out_n, inp, cfg, splits) == binding.OK
        st, ws = _with_plan(L, args, out_w, inp, cfg, splits)
        assert st == binding.OK
        torch.cuda.synchronize()
        if splits == 0:
            assert binding.select_splits(M, N, K, mode, bias, cfg) > 1   # the plan does split
        assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
        nbad, worst, first = compare(out_bits(out_n), ref_mm(inp))
        assert nbad == 0, (nbad, worst, first)


def test_noalloc_plan_beyond_the_scratch_is_refused():
    # 1024 tiles of 256 x 256, 3 splits: 768 MiB of partial tiles > 64 MiB
    L = binding.lib()
    P = 0x10000
    pp = binding.config_names().index("pp_bm256_bn256_bk128_w8_mfma16")
    st = L.fp8_scaled_mm_noalloc(P, P, P, P, None, P, 8192, 8192, 8192, 0, None, pp, 3)
    assert st == binding.ERR_SCRATCH
    assert "scratch" in binding.status_string(st)


def test_noalloc_automatic_plan_shrinks_to_the_scratch():
    # 2048 x 4096 x 14336: the automatic plan is 256 x 256 tiles with 2
    # splits, whose counters and partial tiles (64 MiB + 256 KiB) do not fit
    # the 64 MiB scratch, so the no-alloc call runs the same tiles unsplit:
    # bit-identical to the workspace form with splits = 1, and within the
    # oracle's tolerance.
    L = binding.lib()
    M, N, K = 2048, 4096, 14336
    pp = binding.config_names().index("pp_bm256_bn256_bk128_w8_mfma16")
    assert binding.select_config(M, N, K, RW, False) == pp
    assert binding.select_splits(M, N, K, RW) == 2
    assert binding.workspace_size(M, N, K, RW) > 64 << 20
    inp = wl.make_inputs(M, N, K, RW, "normal", key=577)
    print(f"[noalloc] automatic plan beyond the scratch: shape={inp.shape}", flush=True)
    args = _args(inp)
    out_n = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    out_w = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(L, args, out_n, inp, -1, 0) == binding.OK
    st, _ = _with_plan(L, args, out_w, inp, pp, 1)
    assert st == binding.OK
    torch.cuda.synchronize()
    assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
    nbad, worst, first = compare(out_bits(out_n), ref_mm(inp))
    assert nbad == 0, (nbad, worst, first)
