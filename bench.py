"""Benchmark of the FP8 scaled GEMM on one MI355X.

One step = the whole hot path on the headline workload: the M=N=K=8192
e4m3fn multiply once with per-tensor scales and once with row-wise scales
(inputs N(0,1) -> bf16 -> amax/448 quantised to e4m3fn, B stored N x K,
bf16 out), both already resident in HBM.  `value` is FP8 TFLOP/s over the
timed steps (2*M*N*K per multiply), launched back to back.

Before the warm-up steps the GPU runs the headline launches until about
100 ms of kernel time have passed: under sustained FP8 MFMA load the shader
clock overshoots, then throttles for a few tens of milliseconds, then
settles; the timed steps measure the settled rate.

The JSON line also carries
  roofline      the GEMM kernel's own throughput (algorithmic flops per launch
                over its average launch time: the GPU time between two HIP
                events around the timed steps, on the launch stream, divided
                by the launches) against the dense-FP8 MFMA peak of MI355X;
                config.kernel_us gives the spread of single launches (one
                event pair each, a pass after the timed steps);
  protocol      the gist "matmul_fp8.py" timing protocol (function
                `benchmark`: one untimed call, 8 warm-ups, then 32 runs, each
                timed on its own, reported as p50 with p20 / p80) for both
                headline modes, once with a 1 GiB buffer read before every
                run (the 256 MB MALL holds nothing of the operands) and once
                with the operands left in the caches (the shader clock under
                this load comes from a counter run: GRBM_GUI_ACTIVE per XCD over
                the launch time, in the kernel-trace summary under profiles/);
  cpu_baseline  the CPU oracle timed on this host's cores on one whole step
                (both 8192^3 multiplies, every output element);
  parity        each timed workload's GPU output against that oracle run,
                checked in the CPU-baseline leg: every element of the headline
                outputs, and for the other workloads one whole row in every
                tile row and one whole column in every tile column of the
                launch (the largest error as a fraction of the tolerance);
  secondary     the skinny inference shapes (row-wise + bias, HBM-bound) and
                their 8-way column shards, with the MALL flushed before every
                launch, reported in HBM GB/s; the gist's mid-size shape sweep,
                the ragged shapes and the e5m2 / mixed-format 8192^3 multiplies
                in TFLOP/s, operands resident (us_p50 from an event pair per
                launch; us_batch per launch of 20 back to back, which leaves
                out the few microseconds each event pair adds to a short
                launch); the quantisers in HBM GB/s.  Each multiply names
                the automatic plan it ran ("plan": configuration / splits).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fp8_gemm_pp_sq8192_traffic.txt")
SETTLE_MS = 100.0


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def to_dev(x, dev):
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(dev)


def tile_dims(w):
    """(BM, BN) of the tile configuration the launch uses."""
    import re
    from precision_linear_amd import binding
    name = binding.config_names()[binding.select_config(w.M, w.N, w.K, w.mode, w.bias)]
    return int(re.search(r"bm(\d+)", name).group(1)), int(re.search(r"bn(\d+)", name).group(1))


def covering_indices(n, band, rot):
    """One index in every band of `band` consecutive indices (rotating offset),
    plus the first and the last: with band = the tile height (width), a row
    (column) in every tile row (column) of the grid."""
    idx = [0, n - 1]
    for b in range((n + band - 1) // band):
        lo = b * band
        idx.append(lo + (b * 37 + rot) % min(band, n - lo))
    return np.unique(np.asarray(idx, dtype=np.int64))


class Problem:
    def __init__(self, name, dev):
        import torch
        from precision_linear_amd import workloads as wl
        self.name = name
        self.w = wl.WORKLOADS[name]
        self.inp = wl.make_workload(name)
        i = self.inp
        self.a, self.b = to_dev(i.a, dev), to_dev(i.b, dev)
        self.sa, self.sb = to_dev(i.scale_a, dev), to_dev(i.scale_b, dev)
        self.bias = to_dev(i.bias, dev)
        self.out = torch.empty((self.w.M, self.w.N), dtype=torch.bfloat16, device=dev)
        self.sample = None      # GPU output kept for the parity check

    def launch(self):
        from precision_linear_amd import binding
        binding.fp8_scaled_mm(self.a, self.b, self.sa, self.sb, self.bias, out=self.out,
                              mode=self.w.mode, a_format=self.w.a_format,
                              b_format=self.w.b_format)

    def keep_output(self, full=False):
        """One untimed launch; keeps its output (all of it, or the rows and
        columns of covering_indices) on the host for the parity check."""
        import torch
        self.launch()
        torch.cuda.synchronize()
        bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        if full:
            self.sample = {"full": bits(self.out)}
            return
        bm, bn = tile_dims(self.w)
        rows = covering_indices(self.w.M, bm, len(self.name))
        cols = covering_indices(self.w.N, bn, len(self.name) + 11)
        self.sample = {"rows": rows, "cols": cols,
                       "g_rows": bits(self.out.index_select(0, torch.from_numpy(rows).to(self.out.device))),
                       "g_cols": bits(self.out.index_select(1, torch.from_numpy(cols).to(self.out.device)))}


def plan_of(w):
    """The automatic plan the binding runs for a workload: "configuration
    name / split count" (the binding supplies a workspace, so K may split)."""
    from precision_linear_amd import binding
    c = binding.select_config(w.M, w.N, w.K, w.mode, w.bias, True)
    return f"{binding.config_names()[c]} / {binding.select_splits(w.M, w.N, w.K, w.mode, w.bias)}"


def evict_caches(flush):
    """Read a buffer larger than the 256 MB MALL, so that the next launch finds
    none of its operands in the caches.  (Reading, not writing: dirty lines
    left by a write would be written back during the measured launch.)"""
    import torch
    flush.sum(dtype=torch.int64)


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


def batch_launches(problem, n=20, reps=3):
    """Mean time per launch (ms) of n launches back to back between two HIP
    events, median over reps batches: the kernel's rate without the gaps that
    an event pair around every launch adds."""
    import torch
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            problem.launch()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) / n)
    return sorted(ts)[len(ts) // 2]


def quantiles(ts):
    q = np.quantile(np.asarray(ts, dtype=np.float64), [0.2, 0.5, 0.8])
    return {"p20_us": round(q[0] * 1e3, 2), "p50_us": round(q[1] * 1e3, 2),
            "p80_us": round(q[2] * 1e3, 2), "mean_us": round(float(np.mean(ts)) * 1e3, 2)}


def warm_up(problem, flush=None, min_ms=40.0, max_launches=100):
    """Launches until about min_ms of kernel time has passed (at least 4, at
    most max_launches), so that a timed run of a large multiply meets the
    sustained clock."""
    total = 0.0
    n = 0
    while n < 4 or (total < min_ms and n < max_launches):
        total += sum(time_launches(problem, 4, flush))
        n += 4


def gist_protocol(problem, flush):
    """The gist's `benchmark` timing: one untimed call, 8 warm-ups, 32 runs
    timed one by one (the flush buffer written before every run if given)."""
    problem.launch()
    time_launches(problem, 8, flush)
    ts = time_launches(problem, 32, flush)
    r = quantiles(ts)
    r["tflops_p50"] = round(problem.w.flops / (r["p50_us"] * 1e-6) / 1e12, 1)
    return r


def skinny_results(dev, reps=20, keep=None):
    import torch
    from precision_linear_amd import workloads as wl
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)    # > 256 MB MALL
    res = []
    for name in [n for n in wl.WORKLOADS if n.startswith(("skinny", "shard8"))]:
        p = Problem(name, dev)
        p.keep_output()
        warm_up(p, flush)
        ts = sorted(time_launches(p, reps, flush))
        t50 = ts[len(ts) // 2] * 1e-3
        gbs = p.w.algorithmic_bytes / t50 / 1e9
        res.append({"workload": name, "M": p.w.M, "N": p.w.N, "K": p.w.K,
                    "us_p50": round(t50 * 1e6, 2), "hbm_gbs": round(gbs, 1),
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                    "tflops": round(p.w.flops / t50 / 1e12, 1), "plan": plan_of(p.w),
                    "inputs_sha256": p.inp.sha256()})
        if keep is not None:
            keep.append((name, p.inp, p.sample))
        del p
        torch.cuda.empty_cache()
    return res


QUANT_SHAPES = [(8192, 8192, "rowwise", "e4m3fn"), (8192, 8192, "per_tensor", "e4m3fn"),
                (128, 28672, "rowwise", "e4m3fn"), (8192, 8192, "rowwise", "e5m2")]


def resident_results(dev, names, reps=20, keep=None):
    """Multiplies with operands resident in HBM: TFLOP/s and, against the
    binding roofline max(flops / MFMA peak, bytes / HBM peak), the fraction
    of that bound."""
    import torch
    res = []
    for name in names:
        p = Problem(name, dev)
        p.keep_output()
        warm_up(p)
        ts = sorted(time_launches(p, reps))
        t50 = ts[len(ts) // 2] * 1e-3
        tb = batch_launches(p) * 1e-3
        tf = p.w.flops / t50 / 1e12
        t_mfma = p.w.flops / (PEAK_FP8_TFLOPS * 1e12)
        t_hbm = p.w.algorithmic_bytes / (PEAK_HBM_GBS * 1e9)
        res.append({"workload": name, "M": p.w.M, "N": p.w.N, "K": p.w.K,
                    "formats": f"{p.w.a_format}x{p.w.b_format}",
                    "us_p50": round(t50 * 1e6, 2), "tflops": round(tf, 1),
                    "frac_mfma": round(tf / PEAK_FP8_TFLOPS, 4),
                    "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                    "frac_roofline": round(max(t_mfma, t_hbm) / t50, 4),
                    "us_batch": round(tb * 1e6, 2),
                    "frac_roofline_batch": round(max(t_mfma, t_hbm) / tb, 4),
                    "plan": plan_of(p.w), "inputs_sha256": p.inp.sha256()})
        if keep is not None:
            keep.append((name, p.inp, p.sample))
        del p
        torch.cuda.empty_cache()
    return res


def gist_results(dev, reps=20, keep=None):
    """The gist's mid-size shape sweep (MFMA-bound), operands resident in HBM."""
    from precision_linear_amd import workloads as wl
    return resident_results(dev, [n for n in wl.WORKLOADS if n.startswith("gist")], reps, keep)


def ragged_results(dev, reps=20, keep=None):
    """The ragged shapes (raw e4m3fn codes, log-uniform scales); the K = 32
    and K = 96 ones are bound by the output write."""
    from precision_linear_amd import workloads as wl
    names = [n for n in wl.WORKLOADS if n.startswith("ragged")
             and not (n.startswith("ragged_16384") and n.endswith("rowwise"))]
    return resident_results(dev, names, reps, keep)


def format_results(dev, reps=20, keep=None):
    """8192^3 row-wise with e5m2 operands and with mixed e4m3fn x e5m2."""
    from precision_linear_amd import workloads as wl
    names = [n for n in wl.WORKLOADS if n.startswith("fmt_8192x8192x8192") and n.endswith("rowwise")]
    return resident_results(dev, names, reps, keep)


def vendor_results(dev, reps=20):
    """torch._scaled_mm (hipBLASLt) on the very operands of the headline and
    skinny workloads, timed beside this library's launch with the same
    protocol (skinny: MALL flushed before every launch).  Context only, and
    only with --vendor."""
    import torch
    from precision_linear_amd import workloads as wl
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
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
                vendor(p.bias)
                use_bias = p.bias
            except RuntimeError:
                use_bias = None
                p.bias = None
            entry["bias"] = use_bias is not None

            class V:
                def launch(self):
                    vendor(use_bias)
            warm_up(V(), fl)
            tv = sorted(time_launches(V(), reps, fl))[reps // 2] * 1e-3
            warm_up(p, fl)
            to = sorted(time_launches(p, reps, fl))[reps // 2] * 1e-3
            entry.update({"hipblaslt_us": round(tv * 1e6, 2), "ours_us": round(to * 1e6, 2),
                          "speedup": round(tv / to, 3)})
        except Exception as e:          # hipBLASLt lacks this shape or mode here
            entry["error"] = f"{type(e).__name__}: {str(e)[:160]}"
        res.append(entry)
        del p
        torch.cuda.empty_cache()
    return res


def quant_results(dev, reps=20, keep=None):
    """The dynamic quantiser on seeded N(0,1) bf16 matrices (the producer of A
    and scale_a), with the MALL flushed before every launch.  Algorithmic
    bytes: 2 per input element + 1 per code + 4 per scale.  The per-tensor
    mode reads the input twice (amax pass, then conversion): its bytes count
    once."""
    import torch
    from precision_linear_amd import binding
    from precision_linear_amd import workloads as wl
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    res = []
    for rows, cols, mode, fmt in QUANT_SHAPES:
        bits = wl.bf16_matrix_bits(rows, cols, key=wl.workload_key(f"quant_{rows}x{cols}"))
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
        q, s = binding.fp8_quantize(x, mode, fmt=fmt)
        torch.cuda.synchronize()
        name = f"quantize_{fmt}_{mode}_{rows}x{cols}"
        if keep is not None:
            # row-wise rows are independent: a sample of rows; per-tensor: all
            sel = (np.arange(rows) if mode == "per_tensor"
                   else covering_indices(rows, max(1, rows // 64), len(name)))
            keep.append((name, (bits, mode, fmt, sel),
                         {"q": q.cpu().numpy()[sel], "s": s.cpu().numpy()[sel if mode == "rowwise" else 0]}))
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
        res.append({"workload": name, "rows": rows, "cols": cols,
                    "us_p50": round(t50 * 1e6, 2), "hbm_gbs": round(gbs, 1),
                    "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                    "inputs_sha256": hashlib.sha256(bits.tobytes()).hexdigest()[:16]})
        del x, q, s
        torch.cuda.empty_cache()
    return res


def threads_used():
    try:
        from threadpoolctl import threadpool_info
        return max((d.get("num_threads", 1) for d in threadpool_info()
                    if d.get("user_api") == "blas"), default=1)
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_and_parity(head, kept):
    """The CPU-baseline leg.  The oracle, as it stands, computes one whole
    step (both 8192^3 multiplies, every output element), timed: that is the
    baseline.  Its outputs are then compared with the GPU outputs kept before
    timing (every element), and the oracle also checks the kept rows and
    columns of each secondary workload."""
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare

    def ofmt(f):
        return oracle.E4M3FN if f == "e4m3fn" else oracle.E5M2

    t0 = time.perf_counter()
    refs = {}
    for p in head:
        i = p.inp
        refs[p.name] = oracle.scaled_mm(i.a, i.b, i.scale_a, i.scale_b, i.bias, i.mode)
    dt = time.perf_counter() - t0
    flops = sum(p.w.flops for p in head)
    baseline = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                "cores": int(threads_used()), "kind": "oracle",
                "sample": "one whole step: the 8192^3 multiply per-tensor and row-wise, every "
                          f"output element (fp64 exact accumulation + bf16 RNE), {dt:.1f} s",
                "cpu_model": cpu_model()}
    parity = []
    for p in head:
        nbad, worst, _ = compare(p.sample["full"], refs[p.name])
        parity.append({"workload": p.name, "checked": "every element", "n_bad": nbad,
                       "max_err_over_tol": round(worst, 4)})
    del refs
    for name, inp, smp in kept:
        if name.startswith("quantize"):
            bits, mode, fmt, sel = inp
            om = oracle.PER_TENSOR if mode == "per_tensor" else oracle.ROWWISE
            rq, rs = oracle.quantize(bits[sel] if mode == "rowwise" else bits, om, ofmt(fmt))
            ok = np.array_equal(rq, smp["q"]) and np.array_equal(
                np.asarray(rs).view(np.uint32).ravel(), np.asarray(smp["s"], np.float32).view(np.uint32).ravel())
            parity.append({"workload": name, "checked": f"{len(sel)} rows, bit for bit",
                           "n_bad": 0 if ok else 1, "bitexact": bool(ok)})
            continue
        fa, fb = ofmt(inp.a_format), ofmt(inp.b_format)
        worst_all, nbad_all = 0.0, 0
        for key, kw in (("g_rows", dict(rows=smp["rows"])), ("g_cols", dict(cols=smp["cols"]))):
            ref = oracle.scaled_mm(inp.a, inp.b, inp.scale_a, inp.scale_b, inp.bias, inp.mode,
                                   a_format=fa, b_format=fb, **kw)
            nbad, worst, _ = compare(smp[key], ref)
            nbad_all += nbad
            worst_all = max(worst_all, worst)
        parity.append({"workload": name,
                       "checked": f"{len(smp['rows'])} whole rows, {len(smp['cols'])} whole columns "
                                  "(one in every tile row / column)",
                       "n_bad": nbad_all, "max_err_over_tol": round(worst_all, 4)})
    return baseline, parity


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle leg (baseline and parity checks)")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch._scaled_mm (hipBLASLt) on the same operands")
    ap.add_argument("--profile-gemm", type=int, default=0, metavar="N",
                    help="only launch one workload's multiply N times (counter runs)")
    ap.add_argument("--profile-workload", default="sq8192_pt", metavar="NAME",
                    help="the workload --profile-gemm launches (default: the M=N=K=8192 "
                         "per-tensor multiply)")
    ap.add_argument("--profile-flush", action="store_true",
                    help="with --profile-gemm: write a 1 GiB buffer before every launch so "
                         "the operands come from HBM")
    ap.add_argument("--profile-quant", type=int, default=0, metavar="N",
                    help="only run each quantiser shape of the secondary list N times, the "
                         "MALL flushed before every launch (kernel traces)")
    ap.add_argument("--profile-copy-mib", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB (counter calibration)")
    ap.add_argument("--profile-vendor", type=int, default=0, metavar="R",
                    help="only time the M=N=K=8192 multiplies (per-tensor, row-wise) against "
                         "torch._scaled_mm (hipBLASLt) on the same operands: 60 settling "
                         "launches of each, then R rounds of 40 back-to-back launches of each "
                         "(counter runs and context)")
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
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
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
    if args.profile_vendor:
        from precision_linear_amd import workloads as wl
        res = {}
        for name in ("sq8192_pt", "sq8192_rw"):
            p = Problem(name, dev)
            a8, b8 = p.a.view(torch.float8_e4m3fn), p.b.view(torch.float8_e4m3fn)
            sa, sb = ((p.sa.view(-1, 1), p.sb.view(1, -1)) if p.w.mode == wl.ROWWISE
                      else (p.sa, p.sb))
            fns = {"ours": p.launch,
                   "hipblaslt": lambda: torch._scaled_mm(a8, b8.t(), scale_a=sa, scale_b=sb,
                                                         out_dtype=torch.bfloat16)}
            for f in fns.values():
                for _ in range(60):
                    f()
            torch.cuda.synchronize()
            res[name] = {k: [] for k in fns}
            for _ in range(args.profile_vendor):
                for k, f in fns.items():
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(40):
                        f()
                    e1.record()
                    torch.cuda.synchronize()
                    res[name][k].append(round(e0.elapsed_time(e1) / 40 * 1e3, 1))
            del p
            torch.cuda.empty_cache()
        print(json.dumps({"us_per_launch": res}))
        return
    if args.profile_gemm:
        p = Problem(args.profile_workload, dev)
        flush = (torch.empty(1 << 30, dtype=torch.uint8, device=dev)
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
    for p in probs:                       # the first call of each; outputs kept for parity
        p.keep_output(full=not args.no_cpu)

    # clock settling, then the warm-up steps (all untimed): chunks of 16
    # steps launched back to back, until SETTLE_MS of GPU time has passed
    settle_ms, settle_steps = 0.0, 0
    while settle_ms < SETTLE_MS and settle_steps < 512:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(16):
            for p in probs:
                p.launch()
        e1.record()
        torch.cuda.synchronize()
        settle_ms += e0.elapsed_time(e1)
        settle_steps += 16
    for _ in range(args.warmup):
        for p in probs:
            p.launch()
    torch.cuda.synchronize()

    # The timed steps: launches back to back, with one HIP event pair around
    # all of them on the launch stream (events between launches would add
    # their own gaps to the step time).
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    g0.record()
    for _ in range(args.steps):
        for p in probs:
            p.launch()
    g1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    kernel_avg_s = g0.elapsed_time(g1) * 1e-3 / (args.steps * len(probs))
    achieved = probs[0].w.flops / kernel_avg_s / 1e12
    # Per-launch spread, from one event pair per launch in a pass of its own.
    pairs = {p.name: [] for p in probs}
    for _ in range(args.steps):
        for p in probs:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            p.launch()
            e.record()
            pairs[p.name].append((s, e))
    torch.cuda.synchronize()
    per_kernel = {k: [s.elapsed_time(e) for s, e in v] for k, v in pairs.items()}

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
                   "settle_ms_before_warmup": round(settle_ms, 1),
                   "settle_steps_before_warmup": settle_steps,
                   "kernel_us": {k: quantiles(v) for k, v in per_kernel.items()},
                   "inputs_sha256": {p.name: p.inp.sha256() for p in probs}},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_note": "FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated: bytes "
                                     "the L2s exchange with the fabric (MALL hits included)"},
    }
    print(f"[bench] headline: {value:.1f} TFLOP/s over {args.steps} steps", file=sys.stderr,
          flush=True)

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    line["protocol"] = {
        "runs": "1 untimed + 8 warm-up + 32 timed, one HIP event pair each",
        "flushed": {p.name: gist_protocol(p, flush) for p in probs},
        "resident": {p.name: gist_protocol(p, None) for p in probs},
    }
    del flush
    torch.cuda.empty_cache()

    kept = []
    if not args.no_secondary:
        sec = []
        for part in (skinny_results, gist_results, ragged_results, format_results, quant_results):
            t = time.perf_counter()
            sec += part(dev, keep=kept)
            print(f"[bench] {part.__name__}: {time.perf_counter() - t:.1f} s", file=sys.stderr,
                  flush=True)
        line["secondary"] = sec
    if args.vendor:
        line["vendor"] = vendor_results(dev)
    if not args.no_cpu:
        t = time.perf_counter()
        line["cpu_baseline"], line["parity"] = cpu_baseline_and_parity(probs, kept)
        print(f"[bench] cpu_baseline + parity: {time.perf_counter() - t:.1f} s", file=sys.stderr,
              flush=True)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
