"""Benchmark of the FP8 scaled GEMM on one MI355X.

One step = the whole hot path on the headline workload: the M=N=K=8192
e4m3fn multiply once with per-tensor scales and once with row-wise scales
(inputs N(0,1) -> bf16 -> amax/448 quantised to e4m3fn, B stored N x K,
bf16 out), both already resident in HBM.  `value` is FP8 TFLOP/s over the
timed steps (2*M*N*K per multiply).

The JSON line also carries
  roofline      the GEMM kernel's own throughput (algorithmic flops per launch
                over its average launch time, from HIP events on the launch
                stream) against the dense-FP8 MFMA peak of MI355X;
  cpu_baseline  the CPU oracle timed on a bounded sample (a block of output
                rows of the same problem) on this host's cores;
  secondary     the skinny inference shapes (row-wise + bias, HBM-bound) and
                their 8-way column shards, with the MALL flushed before every
                launch, reported in HBM GB/s; the
                gist's mid-size shape sweep, the ragged shapes and the e5m2 /
                mixed-format 8192^3 multiplies in TFLOP/s; the quantisers in
                HBM GB/s;
  vendor        the same operands through torch._scaled_mm (hipBLASLt on ROCm)
                beside this library's kernel, same timing protocol, for the
                headline and skinny shapes: context, not part of `value`.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 scaled-GEMM TFLOP/s and % of dense-FP8 MFMA peak (per-tensor, row-wise)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "precision_linear_amd", "csrc", "fp8_gemm_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sq8192.txt")


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def to_dev(x, dev):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


class Problem:
    def __init__(self, name, dev):
        from precision_linear_amd import workloads as wl
        self.name = name
        self.w = wl.WORKLOADS[name]
        self.inp = wl.make_workload(name)
        i = self.inp
        self.a, self.b = to_dev(i.a, dev), to_dev(i.b, dev)
        self.sa, self.sb = to_dev(i.scale_a, dev), to_dev(i.scale_b, dev)
        self.bias = to_dev(i.bias, dev)
        import torch
        self.out = torch.empty((self.w.M, self.w.N), dtype=torch.bfloat16, device=dev)

    def launch(self):
        from precision_linear_amd import binding
        binding.fp8_scaled_mm(self.a, self.b, self.sa, self.sb, self.bias, out=self.out,
                              mode=self.w.mode, a_format=self.w.a_format,
                              b_format=self.w.b_format)


def cpu_baseline(problem, target_s=12.0):
    """The oracle, as it stands, on a block of output rows of the same problem."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max((d.get("num_threads", 1) for d in threadpool_info()
                     if d.get("user_api") == "blas"), default=1)
    except Exception:
        cores = os.cpu_count() or 1
    i = problem.inp
    M, N, K = i.shape
    rows = 16
    while True:
        t0 = time.perf_counter()
        oracle.scaled_mm(i.a, i.b, i.scale_a, i.scale_b, i.bias, i.mode, rows=np.arange(rows))
        dt = time.perf_counter() - t0
        if dt * 4 > target_s or rows >= M:
            break
        rows = min(M, int(rows * max(2.0, min(8.0, target_s / max(dt, 1e-3) / 2))))
    tflops = 2.0 * rows * N * K / dt / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{problem.name}: output rows 0..{rows - 1} of {M} (all {N} columns, "
                      f"K={K}), fp64 exact accumulation + bf16 RNE, {dt:.1f} s"}


def evict_caches(flush):
    """Read (not write) a buffer larger than the 256 MB MALL so the next launch
    finds its operands in HBM.  Writing would leave dirty lines whose write-back
    would then be charged to the measured kernel."""
    flush.sum(dtype=torch_int64())


def torch_int64():
    import torch
    return torch.int64


def time_launches(problem, n, flush=None):
    """Per-launch HIP events on the launch stream; returns durations in ms."""
    import torch
    evs = []
    for _ in range(n):
        if flush is not None:
            evict_caches(flush)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        problem.launch()
        e.record()
        evs.append((s, e))
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in evs]


def warm_up(problem, flush=None, min_ms=40.0, max_launches=100):
    """Launches until about min_ms of kernel time has passed (at least 4, at
    most max_launches), so that a timed run of a large multiply meets the
    sustained clock, not the overshoot and throttle of the first tens of
    milliseconds under load."""
    total = 0.0
    n = 0
    while n < 4 or (total < min_ms and n < max_launches):
        total += sum(time_launches(problem, 4, flush))
        n += 4


def skinny_results(dev, reps=20):
    import torch
    from precision_linear_amd import workloads as wl
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)    # > 256 MB MALL
    res = []
    for name in [n for n in wl.WORKLOADS if n.startswith(("skinny", "shard8"))]:
        p = Problem(name, dev)
        warm_up(p, flush)
        ts = sorted(time_launches(p, reps, flush))
        t50 = ts[len(ts) // 2] * 1e-3
        gbs = p.w.algorithmic_bytes / t50 / 1e9
        res.append({"workload": name, "M": p.w.M, "N": p.w.N, "K": p.w.K,
                    "us_p50": round(t50 * 1e6, 2), "hbm_gbs": round(gbs, 1),
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                    "tflops": round(p.w.flops / t50 / 1e12, 1)})
        del p
        torch.cuda.empty_cache()
    return res


QUANT_SHAPES = [(8192, 8192, "rowwise", "e4m3fn"), (8192, 8192, "per_tensor", "e4m3fn"),
                (128, 28672, "rowwise", "e4m3fn"), (8192, 8192, "rowwise", "e5m2")]


def resident_results(dev, names, reps=20):
    """Multiplies with operands resident in HBM: TFLOP/s and, against the
    binding roofline max(flops / MFMA peak, bytes / HBM peak), the fraction
    of that bound."""
    import torch
    from precision_linear_amd import workloads as wl
    res = []
    for name in names:
        p = Problem(name, dev)
        warm_up(p)
        ts = sorted(time_launches(p, reps))
        t50 = ts[len(ts) // 2] * 1e-3
        tf = p.w.flops / t50 / 1e12
        t_mfma = p.w.flops / (PEAK_FP8_TFLOPS * 1e12)
        t_hbm = p.w.algorithmic_bytes / (PEAK_HBM_GBS * 1e9)
        res.append({"workload": name, "M": p.w.M, "N": p.w.N, "K": p.w.K,
                    "formats": f"{p.w.a_format}x{p.w.b_format}",
                    "us_p50": round(t50 * 1e6, 2), "tflops": round(tf, 1),
                    "frac_mfma": round(tf / PEAK_FP8_TFLOPS, 4),
                    "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                    "frac_roofline": round(max(t_mfma, t_hbm) / t50, 4)})
        del p
        torch.cuda.empty_cache()
    return res


def gist_results(dev, reps=20):
    """The gist's mid-size shape sweep (MFMA-bound), operands resident in HBM."""
    from precision_linear_amd import workloads as wl
    return resident_results(dev, [n for n in wl.WORKLOADS if n.startswith("gist")], reps)


def ragged_results(dev, reps=20):
    """The ragged shapes (raw e4m3fn codes, log-uniform scales); the K = 32
    and K = 96 ones are bound by the output write."""
    from precision_linear_amd import workloads as wl
    names = [n for n in wl.WORKLOADS if n.startswith("ragged")
             and not (n.startswith("ragged_16384") and n.endswith("rowwise"))]
    return resident_results(dev, names, reps)


def format_results(dev, reps=20):
    """8192^3 row-wise with e5m2 operands and with mixed e4m3fn x e5m2."""
    from precision_linear_amd import workloads as wl
    names = [n for n in wl.WORKLOADS if n.startswith("fmt_8192x8192x8192") and n.endswith("rowwise")]
    return resident_results(dev, names, reps)


def vendor_results(dev, reps=20):
    """torch._scaled_mm (hipBLASLt) on the very operands of the headline and
    skinny workloads, timed beside this library's launch with the same
    protocol (skinny: MALL flushed before every launch).  Where hipBLASLt
    refuses a bias with row-wise scales, both sides run without the bias."""
    import torch
    from precision_linear_amd import workloads as wl
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    names = ["sq8192_pt", "sq8192_rw"] + [n for n in wl.WORKLOADS
                                          if n.startswith(("skinny", "shard8"))]
    res = []
    for name in names:
        p = Problem(name, dev)
        fl = flush if name.startswith(("skinny", "shard8")) else None
        a8 = p.a.view(torch.float8_e4m3fn)
        b8 = p.b.view(torch.float8_e4m3fn)
        if p.w.mode == wl.ROWWISE:
            sa, sb = p.sa.view(-1, 1), p.sb.view(1, -1)
        else:
            sa, sb = p.sa, p.sb
        entry = {"workload": name, "library": "torch._scaled_mm (hipBLASLt)"}

        def vendor(bias):
            return torch._scaled_mm(a8, b8.t(), scale_a=sa, scale_b=sb, bias=bias,
                                    out_dtype=torch.bfloat16)
        try:
            try:
                ref = vendor(p.bias)
                use_bias = p.bias
            except RuntimeError:
                use_bias = None
                ref = vendor(None)
                p.bias = None
            entry["bias"] = use_bias is not None

            class V:
                def launch(self):
                    vendor(use_bias)
            warm_up(V(), fl)
            tv = sorted(time_launches(V(), reps, fl))[reps // 2] * 1e-3
            warm_up(p, fl)
            to = sorted(time_launches(p, reps, fl))[reps // 2] * 1e-3
            torch.cuda.synchronize()
            diff = (ref.float() - p.out.float()).abs().max().item()
            scale = max(ref.float().abs().max().item(), 1e-30)
            entry.update({"hipblaslt_us": round(tv * 1e6, 2), "ours_us": round(to * 1e6, 2),
                          "speedup": round(tv / to, 3),
                          "max_abs_diff_rel": float(f"{diff / scale:.3g}")})
        except Exception as e:          # hipBLASLt lacks this shape or mode here
            entry["error"] = f"{type(e).__name__}: {str(e)[:160]}"
        res.append(entry)
        del p
        torch.cuda.empty_cache()
    return res


def quant_results(dev, reps=20):
    """The dynamic e4m3fn quantiser on seeded N(0,1) bf16 matrices (the producer
    of A and scale_a), with the MALL flushed before every launch.  Algorithmic
    bytes: 2 per input element + 1 per code + 4 per scale.  The per-tensor mode
    reads the input twice (amax pass, then conversion): its bytes count once."""
    import torch
    from precision_linear_amd import binding
    from precision_linear_amd import workloads as wl
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    res = []
    for rows, cols, mode, fmt in QUANT_SHAPES:
        bits = wl.bf16_matrix_bits(rows, cols, key=wl.workload_key(f"quant_{rows}x{cols}"))
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, s = binding.fp8_quantize(x, mode, fmt=fmt)
        evs = []
        for i in range(reps + 3):
            evict_caches(flush)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            binding.fp8_quantize(x, mode, q=q, scale=s, fmt=fmt)
            e1.record()
            if i >= 3:
                evs.append((e0, e1))
        torch.cuda.synchronize()
        ts = sorted(a.elapsed_time(b) for a, b in evs)
        t50 = ts[len(ts) // 2] * 1e-3
        nbytes = 3 * rows * cols + 4 * (rows if mode == "rowwise" else 1)
        gbs = nbytes / t50 / 1e9
        res.append({"workload": f"quantize_{fmt}_{mode}_{rows}x{cols}", "rows": rows, "cols": cols,
                    "us_p50": round(t50 * 1e6, 2), "hbm_gbs": round(gbs, 1),
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
        del x, q, s
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # Under sustained FP8 MFMA load the MI355X shader clock first overshoots,
    # then throttles (8192^3 launches near 0.48 ms) and settles at its sustained
    # level after about 100 launches (~35 ms, launches near 0.35 ms).  The
    # default warm-up (120 launches) covers that transient, so the timed steps
    # measure the sustained rate.
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=60)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip the skinny shapes")
    ap.add_argument("--profile-gemm", type=int, default=0, metavar="N",
                    help="only launch one workload's multiply N times (counter runs)")
    ap.add_argument("--profile-workload", default="sq8192_pt", metavar="NAME",
                    help="the workload --profile-gemm launches (default: the M=N=K=8192 "
                         "per-tensor multiply)")
    ap.add_argument("--profile-flush", action="store_true",
                    help="with --profile-gemm: read a 1 GiB buffer before every launch so "
                         "the operands come from HBM")
    ap.add_argument("--profile-quant", type=int, default=0, metavar="N",
                    help="only run each quantiser shape of the secondary list N times, the "
                         "MALL flushed before every launch (kernel traces)")
    ap.add_argument("--profile-copy-mib", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the "
              "multiply would shard by output columns, with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from precision_linear_amd import binding

    dev = "cuda:0"
    torch.cuda.set_device(0)
    binding.lib()
    if args.profile_copy_mib:
        src = torch.ones(args.profile_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": src.numel()}))
        return
    if args.profile_quant:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        from precision_linear_amd import workloads as wl
        for rows, cols, mode, fmt in QUANT_SHAPES:
            bits = wl.bf16_matrix_bits(rows, cols, key=wl.workload_key(f"quant_{rows}x{cols}"))
            x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
            q, s = binding.fp8_quantize(x, mode, fmt=fmt)
            for _ in range(args.profile_quant):
                evict_caches(flush)
                binding.fp8_quantize(x, mode, q=q, scale=s, fmt=fmt)
            torch.cuda.synchronize()
        print(json.dumps({"quantiser_launches": args.profile_quant, "shapes": len(QUANT_SHAPES)}))
        return
    if args.profile_gemm:
        p = Problem(args.profile_workload, dev)
        flush = (torch.ones(1 << 30, dtype=torch.uint8, device=dev)
                 if args.profile_flush else None)
        for _ in range(args.profile_gemm):
            if flush is not None:
                evict_caches(flush)
            p.launch()
        torch.cuda.synchronize()
        print(json.dumps({"launches": args.profile_gemm, "workload": p.name,
                          "flush": flush is not None}))
        return
    probs = [Problem("sq8192_pt", dev), Problem("sq8192_rw", dev)]
    flops_step = sum(p.w.flops for p in probs)

    for _ in range(args.warmup):
        for p in probs:
            p.launch()
    torch.cuda.synchronize()

    durations = {p.name: [] for p in probs}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for p in probs:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            p.launch()
            e.record()
            durations[p.name].append((s, e))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    per_kernel = {k: [s.elapsed_time(e) for s, e in v] for k, v in durations.items()}
    avg_ms = {k: sum(v) / len(v) for k, v in per_kernel.items()}
    all_ms = [x for v in per_kernel.values() for x in v]
    kernel_avg_s = sum(all_ms) / len(all_ms) * 1e-3
    achieved = probs[0].w.flops / kernel_avg_s / 1e12

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    tr[k.strip()] = v.strip()
        if tr.get("kernel_sha") == kernel_sha():     # counters taken on this very kernel
            traffic = int(tr["bytes_per_launch"])

    value = flops_step * args.steps / elapsed / 1e12
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn x fp8_e4m3fn -> fp32 acc -> bf16",
        "data": "synthetic (seeded N(0,1) -> bf16 -> amax/448 e4m3fn quantisation)",
        "config": {"workload": "fp8_scaled_mm M=N=K=8192, per-tensor then row-wise, TN, bf16 out",
                   "M": 8192, "N": 8192, "K": 8192, "modes": ["per_tensor", "rowwise"],
                   "tile_config": binding.config_names()[binding.select_config(8192, 8192, 8192, 0)],
                   "frac_of_peak": round(value / PEAK_FP8_TFLOPS, 4),
                   "kernel_ms": {k: round(v, 4) for k, v in avg_ms.items()}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic},
    }
    print(f"[bench] headline: {value:.1f} TFLOP/s over {args.steps} steps", file=sys.stderr,
          flush=True)
    if not args.no_secondary:
        sec = []
        for part in (skinny_results, gist_results, ragged_results, format_results, quant_results):
            t = time.perf_counter()
            sec += part(dev)
            print(f"[bench] {part.__name__}: {time.perf_counter() - t:.1f} s", file=sys.stderr,
                  flush=True)
        line["secondary"] = sec
        t = time.perf_counter()
        line["vendor"] = vendor_results(dev)
        print(f"[bench] vendor_results: {time.perf_counter() - t:.1f} s", file=sys.stderr,
              flush=True)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(probs[0])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
