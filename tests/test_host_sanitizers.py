"""The C ABI's host logic under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the library is rebuilt with the host code of its C-ABI units
instrumented (device code unchanged), and the ABI tests -- argument
validation of every entry point, plan, split and workspace arithmetic,
status strings, the quantiser's checks, the no-device error path -- run
against that build in a child process with the sanitizer runtime preloaded.
Any sanitizer report fails the test."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_abi_tests_under_asan_and_ubsan(tmp_path):
    rt = _runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no hipcc / sanitizer runtime")
    sys.path.insert(0, ROOT)
    from precision_linear_amd import build
    lib = build.build(sanitize=True, out=str(tmp_path / "libfp8_scaled_mm_san.so"))
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    code = (
        "import sys; sys.path.insert(0, %r); sys.path.insert(0, %r)\n"
        "from precision_linear_amd import binding\n"
        "binding.library_path = %r\n"
        "import pytest\n"
        "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', %r]))\n"
    ) % (ROOT, os.path.join(ROOT, "tests"), lib, os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=str(tmp_path), timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    import re
    m = re.search(r"(\d+) passed", r.stdout)
    assert m and int(m.group(1)) >= 50, r.stdout[-2000:]
