"""The exact C entry point of the method, fp8_scaled_mm(A, B, scale_a,
scale_b, bias_or_null, out, M, N, K, scaling_mode, stream), called through
ctypes with raw device pointers (no binding logic in between), against the
oracle on every output element; and its first call on a fresh stream,
captured into a HIP graph."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from precision_linear_amd import binding
from precision_linear_amd import workloads as wl
from parity import compare
from test_gpu_parity import _to_dev, out_bits, ref_mm

pytestmark = pytest.mark.gpu
PT, RW = wl.PER_TENSOR, wl.ROWWISE


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _call(L, args, out, inp, stream):
    a, b, sa, sb, bias = args
    M, N, K = inp.shape
    return L.fp8_scaled_mm(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), _ptr(bias), _ptr(out),
                           M, N, K, inp.mode, ctypes.c_void_p(stream))


@pytest.mark.parametrize("name", ["sq8192_pt", "sq8192_rw", "sq2048_rw", "skinny_m128_k28672_n8192",
                                  "skinny_m16_k28672_n8192", "shard8_m64_k28672_n1024",
                                  "ragged_4095x4097x96_per_tensor", "ragged_8191x1000x4160_rowwise"])
def test_exact_entry_point_full_compare(name):
    inp = wl.make_workload(name)
    M, N, K = inp.shape
    print(f"[abi] fp8_scaled_mm {name} shape={inp.shape}", flush=True)
    args = [_to_dev(x) for x in (inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias)]
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    L = binding.lib()
    st = _call(L, args, out, inp, torch.cuda.current_stream().cuda_stream)
    assert st == binding.OK, binding.status_string(st)
    torch.cuda.synchronize()
    nbad, worst, first = compare(out_bits(out), ref_mm(inp))
    print(f"[abi] worst error {worst:.3f} of the bound", flush=True)
    assert nbad == 0, (nbad, worst, first)


def test_first_calls_on_a_fresh_stream_captured():
    # The very first calls on a stream that has never run one: the plain
    # entry point (no workspace, so no split) and the with-workspace form
    # splitting K into a caller workspace, both captured into one graph, then
    # replayed with eager work in between; every replay gives the bits of the
    # eager calls (made on another stream, with another workspace).
    L = binding.lib()
    inp = wl.make_inputs(64, 2048, 8192, RW, "skinny", bias=True, key=7)
    M, N, K = inp.shape
    cfg = binding.select_config(M, N, K, RW, True, with_workspace=True)
    splits = binding.select_splits(M, N, K, RW, True)
    assert splits > 1
    args = [_to_dev(x) for x in (inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias)]
    need = binding.workspace_size(M, N, K, RW, True, cfg, splits)
    ws_graph = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = [torch.empty(M, N, dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def split_call(out, ws, stream):
        a, b, sa, sb, bias = args
        return L.fp8_scaled_mm_with_plan(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), _ptr(bias), _ptr(out),
                                         M, N, K, RW, ctypes.c_void_p(stream), -1, 0, _ptr(ws),
                                         ws.numel())

    fresh = torch.cuda.Stream()
    fresh.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=fresh):
        assert _call(L, args, outs[0], inp, fresh.cuda_stream) == binding.OK
        assert split_call(outs[1], ws_graph, fresh.cuda_stream) == binding.OK
    torch.cuda.synchronize()

    e_plain = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    e_split = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    cur = torch.cuda.current_stream().cuda_stream
    assert _call(L, args, e_plain, inp, cur) == binding.OK
    assert split_call(e_split, ws_eager, cur) == binding.OK
    torch.cuda.synchronize()
    ref = ref_mm(inp)
    assert compare(out_bits(e_plain), ref)[0] == 0
    assert compare(out_bits(e_split), ref)[0] == 0

    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        junk = torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), e_plain.view(torch.int16)), f"replay {rep}: plain"
        assert torch.equal(outs[1].view(torch.int16), e_split.view(torch.int16)), f"replay {rep}: split"
        del junk
    assert int(ws_graph[:262144].sum()) == 0     # arrival counters back at zero


def test_split_request_without_workspace_is_refused():
    inp = wl.make_inputs(64, 512, 4096, PT, "codes", key=3)
    M, N, K = inp.shape
    args = [_to_dev(x) for x in (inp.a, inp.b, inp.scale_a, inp.scale_b)]
    out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    L = binding.lib()
    a, b, sa, sb = args
    st = L.fp8_scaled_mm_with_plan(_ptr(a), _ptr(b), _ptr(sa), _ptr(sb), None, _ptr(out), M, N, K,
                                   PT, None, -1, 4, None, 0)
    assert st == binding.ERR_WORKSPACE
