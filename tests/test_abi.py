"""Host-side checks of the C ABI: the library loads without a GPU, exports
every function the header declares, and rejects bad arguments before
touching the device."""
import ctypes
import os
import re

import pytest

from precision_linear_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("fp8_scaled_mm.h", "fp8_quantize.h")]


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.library_path):
        from precision_linear_amd import build
        build.build()
    return binding.lib()


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(fp8(?:mm)?_\w+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function(L):
    names = _declared_functions()
    assert len(names) >= 9 and "fp8_quantize_e4m3" in names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(binding.EXPORTS)


def test_status_strings(L):
    for s in range(11):
        assert binding.status_string(s) != "unknown status"
        assert L.fp8mm_status_string(s) == L.fp8_scaled_mm_status_string(s)
    assert binding.status_string(99) == "unknown status"
    assert L.fp8mm_status_string(99) == b"unknown status"


def test_configs_listed(L):
    names = binding.config_names()
    assert len(names) >= 3 and all(names)
    assert L.fp8_scaled_mm_config_name(len(names)) == b""
    assert L.fp8_scaled_mm_config_name(-1) == b""


P = 0x10000          # a 64 KiB-aligned fake device address, never dereferenced


def call(L, A=P, B=P, sa=P, sb=P, bias=None, out=P, M=64, N=64, K=64, mode=0, cfg=-1):
    return L.fp8_scaled_mm_with_config(A, B, sa, sb, bias, out, M, N, K, mode, None, cfg)


@pytest.mark.parametrize("kw,code", [
    (dict(A=None), binding.ERR_NULL), (dict(B=None), binding.ERR_NULL),
    (dict(sa=None), binding.ERR_NULL), (dict(sb=None), binding.ERR_NULL),
    (dict(out=None), binding.ERR_NULL),
    (dict(mode=2), binding.ERR_MODE), (dict(mode=-1), binding.ERR_MODE),
    (dict(M=-1), binding.ERR_SHAPE), (dict(N=-5), binding.ERR_SHAPE),
    (dict(M=2 ** 31), binding.ERR_SHAPE), (dict(K=8), binding.ERR_SHAPE),
    (dict(K=0), binding.ERR_SHAPE), (dict(K=40), binding.ERR_SHAPE),
    (dict(K=2 ** 23 + 16), binding.ERR_SHAPE),
    (dict(A=P + 8), binding.ERR_ALIGN), (dict(B=P + 4), binding.ERR_ALIGN),
    (dict(sa=P + 2), binding.ERR_ALIGN), (dict(sb=P + 1), binding.ERR_ALIGN),
    (dict(out=P + 1), binding.ERR_ALIGN), (dict(bias=P + 1), binding.ERR_ALIGN),
    (dict(cfg=10 ** 6), binding.ERR_CONFIG),
])
def test_validation_errors(L, kw, code):
    assert call(L, **kw) == code


def test_empty_output_is_a_noop(L):
    # M == 0 or N == 0 returns before any device call
    assert call(L, M=0) == binding.OK
    assert call(L, N=0) == binding.OK
    assert call(L, A=None, B=None, sa=None, sb=None, out=None, M=0) == binding.OK
    assert call(L, M=0, K=24) == binding.ERR_SHAPE


def test_no_device_reported():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present: this case would launch on fake pointers")
    L = binding.lib()
    assert call(L) == binding.ERR_DEVICE


def test_select_config_host_logic(L):
    n = L.fp8_scaled_mm_num_configs()
    for shape in [(8192, 8192, 8192), (2048, 2048, 2048), (256, 256, 256), (16, 28672, 8192),
                  (64, 8192, 28672), (128, 28672, 8192), (4095, 4097, 96), (1, 1, 16)]:
        for mode in (0, 1):
            for ws in (0, 1):
                c = L.fp8_scaled_mm_select_config(*shape, mode, 1, ws)
                assert 0 <= c < n
    assert L.fp8_scaled_mm_select_config(16, 16, 16, 3, 0, 0) == -1
    assert L.fp8_scaled_mm_select_config(16, 16, 24, 0, 0, 1) == -1


def test_grid_size_is_persistent(L):
    n = L.fp8_scaled_mm_num_configs()
    for c in range(n):
        g = L.fp8_scaled_mm_grid_size(c, 8192, 8192, 256)
        assert g in (256, 512, 768)   # persistent: one, two or three workgroups per CU
        assert L.fp8_scaled_mm_grid_size(c, 1, 1, 256) == 1
    assert L.fp8_scaled_mm_grid_size(0, 0, 5, 256) == 0


def test_python_binding_rejects_bad_tensors():
    import torch
    a = torch.zeros(4, 32, dtype=torch.float32)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, a, a, a)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, a, a, a, mode="columnwise")


def test_workspace_and_split_host_logic(L):
    # a grid that fills the GPU needs no split and no workspace
    assert L.fp8_scaled_mm_select_splits(8192, 8192, 8192, 0, 0, -1) == 1
    assert L.fp8_scaled_mm_workspace_size(8192, 8192, 8192, 0, 0, -1, 0) == 0
    # a few tiles with a long K split, and the workspace covers counters + partials
    cfg = binding.config_names().index("bm128_bn128_bk128_w2x2_s2_mfma32")
    s = L.fp8_scaled_mm_select_splits(128, 8192, 28672, 1, 1, cfg)
    assert s > 1
    ws = L.fp8_scaled_mm_workspace_size(128, 8192, 28672, 1, 1, cfg, s)
    tiles = 1 * 64
    assert ws >= tiles * s * 128 * 128 * 4 + tiles * 4
    # explicit split counts are clamped to the number of K slices
    assert L.fp8_scaled_mm_workspace_size(128, 128, 256, 0, 0, cfg, 8) == \
        L.fp8_scaled_mm_workspace_size(128, 128, 256, 0, 0, cfg, 2)
    assert L.fp8_scaled_mm_select_splits(16, 16, 16, 5, 0, -1) == -1


def test_stream_k_plan_validation(L):
    P = 0x10000
    f = L.fp8_scaled_mm_with_plan
    names = binding.config_names()
    c9 = names.index("bm128_bn128_bk128_w2x2_s2_mfma32")
    pp = names.index("pp_bm256_bn256_bk128_w8_mfma16")
    sk = binding.SPLITS_STREAM_K
    # a workspace is required; the ping-pong kernel and configurations that
    # cannot split K have no stream-K form; -2 is no plan at all
    assert f(P, P, P, P, None, P, 512, 3072, 12288, 1, None, c9, sk, None, 0) == binding.ERR_WORKSPACE
    assert f(P, P, P, P, None, P, 512, 3072, 12288, 1, None, pp, sk, P, 1 << 30) == binding.ERR_CONFIG
    assert f(P, P, P, P, None, P, 512, 3072, 12288, 1, None, c9, -2, P, 1 << 30) == binding.ERR_CONFIG
    assert L.fp8_scaled_mm_workspace_size(512, 3072, 12288, 1, 0, pp, sk) == 0
    for cfg in range(len(names)):
        # a configuration without a split-K form has no stream-K form either
        if cfg != pp and L.fp8_scaled_mm_workspace_size(512, 3072, 12288, 1, 0, cfg, 2) == 0:
            assert L.fp8_scaled_mm_workspace_size(512, 3072, 12288, 1, 0, cfg, sk) == 0


def test_stream_k_workspace_bound(L):
    # room for the partial tiles of every tile's segments, for any grid of up
    # to 1024 workgroups: 96 tiles of 128 x 128, 96 K slices each
    c9 = binding.config_names().index("bm128_bn128_bk128_w2x2_s2_mfma32")
    ws = L.fp8_scaled_mm_workspace_size(512, 3072, 12288, 1, 0, c9, binding.SPLITS_STREAM_K)
    tiles = 4 * 24
    segs = -(-1024 // tiles) + 1           # workgroups that can meet one tile
    assert ws == 256 * 1024 + tiles * segs * 128 * 128 * 4


def test_plan_validation(L):
    P = 0x10000
    f = L.fp8_scaled_mm_with_plan
    cfg = binding.config_names().index("bm128_bn128_bk128_w2x2_s2_mfma32")
    assert f(P, P, P, P, None, P, 128, 128, 4096, 0, None, cfg, 65, None, 0) == binding.ERR_CONFIG
    assert f(P, P, P, P, None, P, 128, 128, 4096, 0, None, cfg, -2, None, 0) == binding.ERR_CONFIG
    # caller workspace too small for a 4-way split
    assert f(P, P, P, P, None, P, 128, 128, 4096, 0, None, cfg, 4, P, 1024) == binding.ERR_WORKSPACE
    need = L.fp8_scaled_mm_workspace_size(128, 128, 4096, 0, 0, cfg, 4)
    assert f(P, P, P, P, None, P, 128, 128, 4096, 0, None, cfg, 4, P + 128, need) == binding.ERR_ALIGN
    # splitting K needs a caller workspace: the library allocates none
    assert f(P, P, P, P, None, P, 128, 128, 4096, 0, None, cfg, 4, None, 0) == binding.ERR_WORKSPACE
    assert L.fp8_scaled_mm_typed(P, 0, P, 0, P, P, None, P, 128, 128, 4096, 0, None, cfg, 2,
                                 None, 0) == binding.ERR_WORKSPACE


# ---- quantiser ---------------------------------------------------------------

def qcall(L, x=P, q=P, scale=P, rows=64, cols=64, mode=1):
    return L.fp8_quantize_e4m3(x, q, scale, rows, cols, mode, None)


@pytest.mark.parametrize("kw,code", [
    (dict(mode=2), binding.Q_ERR_MODE), (dict(mode=-1), binding.Q_ERR_MODE),
    (dict(cols=24), binding.Q_ERR_SHAPE), (dict(rows=-1), binding.Q_ERR_SHAPE),
    (dict(cols=-16), binding.Q_ERR_SHAPE), (dict(cols=(1 << 31) + 16), binding.Q_ERR_SHAPE),
    (dict(x=None), binding.Q_ERR_NULL), (dict(q=None), binding.Q_ERR_NULL),
    (dict(scale=None), binding.Q_ERR_NULL), (dict(scale=None, rows=0, mode=0), binding.Q_ERR_NULL),
    (dict(x=P + 8), binding.Q_ERR_ALIGN), (dict(q=P + 4), binding.Q_ERR_ALIGN),
    (dict(scale=P + 2), binding.Q_ERR_ALIGN),
])
def test_quantize_rejects_bad_arguments(L, kw, code):
    assert qcall(L, **kw) == code


def test_quantize_empty_rowwise_needs_no_device(L):
    # no rows: nothing at all to do, not even scales
    assert qcall(L, x=None, q=None, rows=0, cols=64, mode=1) == binding.Q_OK
    assert qcall(L, x=None, q=None, scale=None, rows=0, cols=64, mode=1) == binding.Q_OK


def test_quantize_status_strings(L):
    for s in range(8):
        assert L.fp8_quantize_status_string(s) != b"unknown status"
    assert L.fp8_quantize_status_string(42) == b"unknown status"


# ---- operand formats -----------------------------------------------------------

def tcall(L, fa=0, fb=0, M=64, N=64, K=64, mode=0, cfg=-1, A=P, B=P):
    return L.fp8_scaled_mm_typed(A, fa, B, fb, P, P, None, P, M, N, K, mode, None, cfg, 0, None, 0)


@pytest.mark.parametrize("fa,fb", [(2, 0), (0, 2), (-1, 0), (0, -1), (7, 7)])
def test_typed_rejects_unknown_formats(L, fa, fb):
    assert tcall(L, fa, fb) == binding.ERR_FORMAT
    assert tcall(L, fa, fb, M=0) == binding.ERR_FORMAT      # checked before anything else


def test_typed_validates_like_the_plain_entry(L):
    for fa, fb in ((1, 1), (0, 1), (1, 0)):
        assert tcall(L, fa, fb, K=40) == binding.ERR_SHAPE
        assert tcall(L, fa, fb, A=P + 8) == binding.ERR_ALIGN
        assert tcall(L, fa, fb, mode=5) == binding.ERR_MODE
        assert tcall(L, fa, fb, M=0) == binding.OK
        assert tcall(L, fa, fb, cfg=10 ** 6) == binding.ERR_CONFIG
    assert binding.status_string(binding.ERR_FORMAT).startswith("unknown operand format")


def test_python_binding_rejects_bad_formats():
    import torch
    a = torch.zeros(4, 32, dtype=torch.uint8)
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a, a, a, a, a_format="e3m4")
    with pytest.raises(ValueError):
        binding.fp8_scaled_mm(a.view(torch.float8_e5m2), a, a, a, a_format="e4m3fn")
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.fp8_quantize(x, fmt="e4m3")


@pytest.mark.parametrize("kw,code", [
    (dict(mode=2), binding.Q_ERR_MODE), (dict(cols=24), binding.Q_ERR_SHAPE),
    (dict(x=None), binding.Q_ERR_NULL), (dict(q=P + 4), binding.Q_ERR_ALIGN),
])
def test_quantize_e5m2_rejects_bad_arguments(L, kw, code):
    args = dict(x=P, q=P, scale=P, rows=64, cols=64, mode=1)
    args.update(kw)
    assert L.fp8_quantize_e5m2(args["x"], args["q"], args["scale"], args["rows"], args["cols"],
                               args["mode"], None) == code


def test_quantize_workspace_size(L):
    # per-tensor calls with elements take the one-pass kernel's workspace;
    # row-wise and empty calls take none
    assert L.fp8_quantize_workspace_size(8192, 8192, binding.PER_TENSOR) == 67840
    assert L.fp8_quantize_workspace_size(1, 16, binding.PER_TENSOR) == 67840
    assert L.fp8_quantize_workspace_size(8192, 8192, binding.ROWWISE) == 0
    assert L.fp8_quantize_workspace_size(0, 64, binding.PER_TENSOR) == 0
    assert L.fp8_quantize_workspace_size(64, 0, binding.PER_TENSOR) == 0


@pytest.mark.parametrize("fn", ["fp8_quantize_e4m3_ws", "fp8_quantize_e5m2_ws"])
def test_quantize_ws_rejects_bad_workspaces(L, fn):
    f = getattr(L, fn)
    need = L.fp8_quantize_workspace_size(64, 64, binding.PER_TENSOR)
    assert f(P, P, P, 64, 64, binding.PER_TENSOR, P, need - 4, None) == binding.Q_ERR_WORKSPACE
    assert f(P, P, P, 64, 64, binding.PER_TENSOR, P + 2, need, None) == binding.Q_ERR_ALIGN
    # the shared argument checks come first, as in fp8_quantize_e4m3
    assert f(P, P, P, 64, 24, binding.PER_TENSOR, P, need, None) == binding.Q_ERR_SHAPE
    assert f(P, P, P, 64, 64, 2, P, need, None) == binding.Q_ERR_MODE


def test_quantize_wait_limit_hook_returns_the_previous_limit(L):
    assert L.fp8_quantize_set_wait_limit_us(5) == 1000
    assert L.fp8_quantize_set_wait_limit_us(-1) == 5
    assert L.fp8_quantize_set_wait_limit_us(-1) == 1000


# The plans chosen for the benchmarked shapes (by the fixed rules or the plan
# cost model, both from measurements on MI355X): a change to either shows up
# here.
PLANS = {
    (8192, 8192, 8192): ("pp_bm256_bn256_bk128_w8_mfma16", 1),
    (16, 28672, 8192): ("bm16_bn112_bk256_w1x7_s4_mfma16", 1),
    (64, 28672, 8192): ("bm64_bn112_bk256_w1x7_s3_mfma16", 1),
    (128, 28672, 8192): ("bm128_bn128_bk128_w2x4_s4_mfma32", 1),
    (16, 8192, 28672): ("bm16_bn64_bk256_w1x4_s4_mfma16", 2),
    (64, 8192, 28672): ("bm64_bn64_bk256_w1x4_s4_mfma16", 2),
    (128, 8192, 28672): ("bm128_bn128_bk128_w2x4_s4_mfma32", 4),
    (16, 3584, 8192): ("bm16_bn64_bk256_w1x4_s4_mfma16", 4),
    (128, 3584, 8192): ("bm128_bn64_bk256_w4x2_s3_mfma16", 4),
    (16, 1024, 28672): ("bm16_bn32_bk512_w1x2_s6_mfma16", 8),
    (64, 1024, 28672): ("bm64_bn32_bk256_w4x2_s4_mfma16", 8),
    (128, 1024, 28672): ("bm64_bn64_bk256_w1x4_s4_mfma16", 8),
    (512, 12288, 3072): ("bm128_bn128_bk128_w2x2_s2_mfma32", 1),
    (512, 3072, 12288): ("bm128_bn128_bk128_w2x4_s4_mfma32", 2),
    (1152, 3072, 12288): ("bm128_bn128_bk128_w2x4_s4_mfma32", 1),
    (2304, 3072, 12288): ("pp_bm256_bn256_bk128_w8_mfma16", 2),
    (8191, 1000, 4160): ("bm128_bn128_bk128_w2x2_s2_mfma32", 1),
    (4096, 4096, 32): ("pp_bm256_bn256_bk128_w8_mfma16", 1),
    (4095, 4097, 96): ("bm64_bn128_bk128_w2x2_s2_mfma32", 1),
}


@pytest.mark.parametrize("shape", list(PLANS), ids=[f"{m}x{n}x{k}" for m, n, k in PLANS])
def test_plans_of_benchmarked_shapes(L, shape):
    # with a workspace (the binding supplies one when the plan splits K)
    names = binding.config_names()
    M, N, K = shape
    cfg = L.fp8_scaled_mm_select_config(M, N, K, 1, 1, 1)
    assert (names[cfg], L.fp8_scaled_mm_select_splits(M, N, K, 1, 1, -1)) == PLANS[shape]


@pytest.mark.parametrize("shape", list(PLANS), ids=[f"{m}x{n}x{k}" for m, n, k in PLANS])
def test_plans_without_workspace(L, shape):
    # fp8_scaled_mm has no workspace, so it never splits K: its configuration
    # differs from the plan with a workspace only where that plan splits
    M, N, K = shape
    with_ws = L.fp8_scaled_mm_select_config(M, N, K, 1, 1, 1)
    without = L.fp8_scaled_mm_select_config(M, N, K, 1, 1, 0)
    if PLANS[shape][1] == 1:
        assert without == with_ws
    assert 0 <= without < L.fp8_scaled_mm_num_configs()


def _imported_modules(path):
    import ast
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_product_package_never_imports_the_oracle():
    """The oracle is test infrastructure: no module of the package (the path
    every multiply takes) imports it, so no result can come from it."""
    pkg = os.path.join(ROOT, "precision_linear_amd")
    checked = 0
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                mods = list(_imported_modules(os.path.join(dirpath, f)))
                assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), f
                checked += 1
    assert checked >= 4
    for f in os.listdir(os.path.join(pkg, "csrc")):
        text = open(os.path.join(pkg, "csrc", f)).read()
        assert "oracle" not in text, f


def test_missing_library_is_an_error(monkeypatch):
    """Without the HIP library the binding raises instead of computing anything."""
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "library_path", os.path.join(ROOT, "no_such_dir", "lib.so"))
    with pytest.raises(RuntimeError, match="no non-HIP fallback"):
        binding.lib()
    with pytest.raises(RuntimeError, match="missing"):
        binding.select_config(64, 64, 64, "per_tensor")
