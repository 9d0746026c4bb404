"""Builds libfp8_scaled_mm.so (the HIP kernels -- scaled multiply and
quantiser -- and their C ABI) for gfx950.

hipcc cross-compiles without a GPU.  The library is written next to this
file so that it travels with the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
# The host logic and C ABI, one translation unit per operand-format pair of
# the multiply's kernels, and the quantiser.  They compile in parallel.
SRCS = [os.path.join(HERE, "csrc", f) for f in
        ["fp8_scaled_mm.hip"] + [f"fp8_gemm_f{k}.hip" for k in range(4)] + ["fp8_quantize.hip"]]
HEADERS = [os.path.join(HERE, "csrc", "fp8_gemm_kernels.h")]
LIB = os.path.join(HERE, "libfp8_scaled_mm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        sys.stderr.write(res.stderr)


# Host-only sanitizer instrumentation (AddressSanitizer + UndefinedBehavior-
# Sanitizer) for the translation units whose host code is the C ABI's logic
# (argument validation, plan and workspace arithmetic); device code is built
# as usual.  Every -fsanitize flag is scoped to the host compilation.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
HOST_LOGIC_SRCS = {"fp8_scaled_mm.hip", "fp8_quantize.hip"}


def build(verbose: bool = False, sanitize: bool = False, out: str | None = None) -> str:
    """Compile every source to an object (in parallel), then link the
    shared library; always rebuilds.  sanitize=True builds the host logic
    with ASan/UBSan (a test build, loaded with the sanitizer runtime
    preloaded) into `out` instead of the package's library."""
    from concurrent.futures import ThreadPoolExecutor
    target = out or LIB
    objdir = tempfile.mkdtemp(prefix="fp8mm_build_")
    try:
        objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in SRCS]
        jobs = []
        for src, obj in zip(SRCS, objs):
            extra = SANITIZE_HOST if sanitize and os.path.basename(src) in HOST_LOGIC_SRCS else []
            jobs.append([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj])
        workers = max(1, min(len(jobs), os.cpu_count() or 1))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        tmp = target + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", *objs, "-o", tmp], verbose)
        shutil.move(tmp, target)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
