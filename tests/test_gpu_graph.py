"""The library's calls captured into a HIP graph (through torch.cuda.CUDAGraph)
replay to the same bits as the eager calls: they launch kernels only (no host
synchronisation, no allocation, no memset)."""
import numpy as np
import pytest
import torch

from precision_linear_amd import binding
from precision_linear_amd import workloads as wl
from test_gpu_parity import _to_dev

pytestmark = pytest.mark.gpu
PT, RW = wl.PER_TENSOR, wl.ROWWISE


def test_graph_replays_match_eager():
    dev = "cuda:0"
    gen = wl.make_inputs(512, 768, 1024, PT, "codes", key=41)          # one plain tile grid
    spl = wl.make_inputs(128, 1024, 8192, RW, "skinny", bias=True, key=42)   # split over K
    xa = torch.from_numpy(wl.bf16_matrix_bits(256, 4096, key=43).view(np.int16)).view(torch.bfloat16).to(dev)

    g_args = [_to_dev(x) for x in (gen.a, gen.b, gen.scale_a, gen.scale_b)]
    s_args = [_to_dev(x) for x in (spl.a, spl.b, spl.scale_a, spl.scale_b, spl.bias)]
    assert binding.select_splits(128, 1024, 8192, RW, True) > 1
    out_g = torch.empty(512, 768, dtype=torch.bfloat16, device=dev)
    out_s = torch.empty(128, 1024, dtype=torch.bfloat16, device=dev)
    q_rw = torch.empty(256, 4096, dtype=torch.uint8, device=dev)
    s_rw = torch.empty(256, dtype=torch.float32, device=dev)
    q_pt = torch.empty(256, 4096, dtype=torch.uint8, device=dev)
    s_pt = torch.empty(1, dtype=torch.float32, device=dev)

    def calls():
        binding.fp8_scaled_mm(*g_args, out=out_g, mode=PT)
        binding.fp8_scaled_mm(*s_args[:4], s_args[4], out=out_s, mode=RW)
        binding.fp8_quantize(xa, RW, q=q_rw, scale=s_rw)
        binding.fp8_quantize(xa, PT, q=q_pt, scale=s_pt)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                      # eager, on the capture stream (the binding's workspace)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out_g, out_s, q_rw, s_rw, q_pt, s_pt)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        calls()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (out_g, out_s, q_rw, s_rw, q_pt, s_pt):
            t.zero_()
        junk = torch.randn(512, 512, device=dev) @ torch.randn(512, 512, device=dev)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("gemm", "split gemm", "q rw", "s rw", "q pt", "s pt"),
                                   (out_g, out_s, q_rw, s_rw, q_pt, s_pt), eager):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.uint8 else got,
                               want.view(torch.uint8) if want.dtype != torch.uint8 else want), \
                f"replay {rep}: {name} differs from the eager result"
        del junk
