"""ctypes binding of libfp8_scaled_mm.so: argument marshalling only.

Every step of the multiply runs in the HIP library; this module turns torch
tensors into device pointers, sizes and the current stream, and turns
status codes into exceptions.  A missing library is an error (there is no
fallback path).
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libfp8_scaled_mm.so")

PER_TENSOR = 0
ROWWISE = 1
_MODES = {"per_tensor": PER_TENSOR, "tensorwise": PER_TENSOR, "rowwise": ROWWISE,
          PER_TENSOR: PER_TENSOR, ROWWISE: ROWWISE}

# operand formats (enum fp8mm_format)
E4M3FN = 0
E5M2 = 1
_FORMATS = {"e4m3fn": E4M3FN, "e5m2": E5M2, E4M3FN: E4M3FN, E5M2: E5M2}

# splits value of a stream-K plan (FP8MM_SPLITS_STREAM_K in include/fp8_scaled_mm.h)
SPLITS_STREAM_K = -1

# status codes from include/fp8_scaled_mm.h
(OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_DEVICE, ERR_LAUNCH, ERR_CONFIG, ERR_WORKSPACE,
 ERR_FORMAT, ERR_SCRATCH) = range(11)
_ARG_ERRORS = {ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_MODE, ERR_CONFIG, ERR_WORKSPACE, ERR_FORMAT,
               ERR_SCRATCH}

EXPORTS = ("fp8_scaled_mm", "fp8_scaled_mm_with_config", "fp8_scaled_mm_with_plan",
           "fp8_scaled_mm_typed", "fp8_scaled_mm_noalloc",
           "fp8_scaled_mm_workspace_size", "fp8_scaled_mm_select_splits",
           "fp8_scaled_mm_num_configs", "fp8_scaled_mm_config_name", "fp8_scaled_mm_select_config",
           "fp8_scaled_mm_grid_size", "fp8_scaled_mm_status_string", "fp8mm_status_string",
           "fp8_quantize_e4m3", "fp8_quantize_e5m2", "fp8_quantize_e4m3_ws", "fp8_quantize_e5m2_ws",
           "fp8_quantize_workspace_size", "fp8_quantize_set_wait_limit_us",
           "fp8_quantize_status_string")

# status codes from include/fp8_quantize.h
(Q_OK, Q_ERR_NULL, Q_ERR_SHAPE, Q_ERR_ALIGN, Q_ERR_MODE, Q_ERR_DEVICE, Q_ERR_LAUNCH,
 Q_ERR_WORKSPACE) = range(8)
_Q_ARG_ERRORS = {Q_ERR_NULL, Q_ERR_SHAPE, Q_ERR_ALIGN, Q_ERR_MODE, Q_ERR_WORKSPACE}


class Fp8MMError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"fp8_scaled_mm failed: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is missing: build it with "
                "`python -m precision_linear_amd.build` (there is no non-HIP fallback)")
        L = ctypes.CDLL(library_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.fp8_scaled_mm.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
        L.fp8_scaled_mm.restype = i32
        L.fp8_scaled_mm_with_config.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32]
        L.fp8_scaled_mm_with_config.restype = i32
        L.fp8_scaled_mm_with_plan.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32,
                                              i32, vp, i64]
        L.fp8_scaled_mm_with_plan.restype = i32
        L.fp8_scaled_mm_typed.argtypes = [vp, i32, vp, i32, vp, vp, vp, vp, i64, i64, i64, i32, vp,
                                          i32, i32, vp, i64]
        L.fp8_scaled_mm_typed.restype = i32
        L.fp8_scaled_mm_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32, i32]
        L.fp8_scaled_mm_noalloc.restype = i32
        L.fp8_scaled_mm_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, i32]
        L.fp8_scaled_mm_workspace_size.restype = i64
        L.fp8_scaled_mm_select_splits.argtypes = [i64, i64, i64, i32, i32, i32]
        L.fp8_scaled_mm_select_splits.restype = i32
        L.fp8_scaled_mm_num_configs.argtypes = []
        L.fp8_scaled_mm_num_configs.restype = i32
        L.fp8_scaled_mm_config_name.argtypes = [i32]
        L.fp8_scaled_mm_config_name.restype = ctypes.c_char_p
        L.fp8_scaled_mm_select_config.argtypes = [i64, i64, i64, i32, i32, i32]
        L.fp8_scaled_mm_select_config.restype = i32
        L.fp8_scaled_mm_grid_size.argtypes = [i32, i64, i64, i32]
        L.fp8_scaled_mm_grid_size.restype = i64
        L.fp8_scaled_mm_status_string.argtypes = [i32]
        L.fp8_scaled_mm_status_string.restype = ctypes.c_char_p
        L.fp8mm_status_string.argtypes = [i32]
        L.fp8mm_status_string.restype = ctypes.c_char_p
        L.fp8_quantize_e4m3.argtypes = [vp, vp, vp, i64, i64, i32, vp]
        L.fp8_quantize_e4m3.restype = i32
        L.fp8_quantize_e5m2.argtypes = [vp, vp, vp, i64, i64, i32, vp]
        L.fp8_quantize_e5m2.restype = i32
        for name in ("fp8_quantize_e4m3_ws", "fp8_quantize_e5m2_ws"):
            getattr(L, name).argtypes = [vp, vp, vp, i64, i64, i32, vp, i64, vp]
            getattr(L, name).restype = i32
        L.fp8_quantize_workspace_size.argtypes = [i64, i64, i32]
        L.fp8_quantize_workspace_size.restype = i64
        L.fp8_quantize_set_wait_limit_us.argtypes = [i64]
        L.fp8_quantize_set_wait_limit_us.restype = i64
        L.fp8_quantize_status_string.argtypes = [i32]
        L.fp8_quantize_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fp8_scaled_mm_status_string(int(status)).decode()


def config_names() -> list:
    L = lib()
    return [L.fp8_scaled_mm_config_name(i).decode() for i in range(L.fp8_scaled_mm_num_configs())]


def select_config(M, N, K, mode, has_bias=False, with_workspace=True) -> int:
    """The automatic configuration; with_workspace=True is the plan this
    module's fp8_scaled_mm runs (it supplies a workspace whenever the plan
    splits K), False the one of the C entry point fp8_scaled_mm."""
    return int(lib().fp8_scaled_mm_select_config(M, N, K, _MODES[mode], int(bool(has_bias)),
                                                 int(bool(with_workspace))))


def select_splits(M, N, K, mode, has_bias=False, config=-1) -> int:
    return int(lib().fp8_scaled_mm_select_splits(M, N, K, _MODES[mode], int(bool(has_bias)),
                                                 int(config)))


def workspace_size(M, N, K, mode, has_bias=False, config=-1, splits=0) -> int:
    return int(lib().fp8_scaled_mm_workspace_size(M, N, K, _MODES[mode], int(bool(has_bias)),
                                                  int(config), int(splits)))


# Split-K workspaces handed to the library, per (device, stream): zero-filled
# torch allocations (the library allocates nothing itself).  Calls on one
# stream are ordered, so they can share one; a larger one replaces it for
# later calls, but none is ever freed, because a captured HIP graph may still
# hold its address.
_workspaces: dict = {}


def _workspace(device: torch.device, stream: int, nbytes: int, kind: str = "mm") -> torch.Tensor:
    key = (device.index, stream, kind)
    have = _workspaces.get(key)
    if have and have[-1].numel() >= nbytes:
        return have[-1]
    size = max(nbytes, 2 * have[-1].numel() if have else 0)
    size = (size + (1 << 20) - 1) >> 20 << 20
    ws = torch.zeros(size, dtype=torch.uint8, device=device)   # a fill kernel on this stream
    _workspaces.setdefault(key, []).append(ws)
    return ws


_TORCH_FORMATS = {torch.float8_e4m3fn: E4M3FN, torch.float8_e5m2: E5M2}


def _as_codes(t: torch.Tensor, name: str, fmt) -> tuple:
    """(uint8 view, format id).  A float8 tensor carries its format; uint8
    codes take `fmt` (default e4m3fn)."""
    dt = t.dtype
    if fmt is None and dt == torch.uint8:
        return t, E4M3FN
    if fmt is not None and fmt not in _FORMATS:
        raise ValueError(f"{name}_format must be 'e4m3fn' or 'e5m2', got {fmt!r}")
    if dt in _TORCH_FORMATS:
        f = _TORCH_FORMATS[dt]
        if fmt is not None and _FORMATS[fmt] != f:
            raise ValueError(f"{name} is {dt} but {name}_format={fmt!r}")
        return t.view(torch.uint8), f
    if dt == torch.uint8:
        return t, _FORMATS[fmt]
    raise ValueError(f"{name} must be float8_e4m3fn, float8_e5m2 or uint8 codes, got {dt}")


def _check_devices(dev: int, tensors) -> None:
    """Every (name, tensor) given (None skipped) must live on GPU `dev`: the
    library passes their pointers to kernels on that device.  Compares
    device indices (a CPU tensor's is -1)."""
    for name, t in tensors:
        if t is not None and t.get_device() != dev:
            raise ValueError(f"{name} is on {t.device}, expected cuda:{dev}")


# The current stream's raw handle for a device index: torch's direct accessor
# where it has one (no Stream object built per call), else the public API.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_of(dev: int) -> int:
    if _raw_stream is not None:
        return _raw_stream(dev)
    return torch.cuda.current_stream(dev).cuda_stream


# Workspace bytes of automatic plans, per (device, M, N, K, mode, bias, config,
# splits): the plan depends on nothing else, so the size is asked once.
_ws_sizes: dict = {}


def fp8_scaled_mm(a: torch.Tensor, b: torch.Tensor, scale_a: torch.Tensor, scale_b: torch.Tensor,
                  bias: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  mode="per_tensor", config: int = -1, splits: int = 0,
                  workspace: torch.Tensor | None = None, a_format=None,
                  b_format=None) -> torch.Tensor:
    """out = bf16(scale_a * scale_b * (a @ b^T) + bias) with a: M x K and b: N x K
    (float8 codes, K contiguous).  b may also be given as a K x N column-major
    view (stride (1, K)), which is the same memory.  Each operand is e4m3fn or
    e5m2: taken from its torch dtype, or from a_format / b_format for uint8
    codes (default e4m3fn).  `config` (-1: automatic) and `splits` (0:
    automatic; SPLITS_STREAM_K: stream-K) select the plan.  When the plan
    splits K, its workspace is
    `workspace` (a GPU byte tensor, zero-filled before first use) or, if that
    is None, one this module keeps per stream (allocated by torch)."""
    m = _MODES.get(mode) if isinstance(mode, (str, int)) else None
    if m is None:
        raise ValueError(f"mode must be 'per_tensor' or 'rowwise', got {mode!r}")
    a, fa = _as_codes(a, "a", a_format)
    b, fb = _as_codes(b, "b", b_format)
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    if b.shape[1] == K and b.is_contiguous():
        N = b.shape[0]
    elif b.shape[0] == K and b.stride() == (1, K):
        b = b.t()
        N = b.shape[0]
    else:
        raise ValueError(f"b must be N x K contiguous or K x N column-major, got {tuple(b.shape)} "
                         f"strides {b.stride()} for K={K}")
    if not a.is_contiguous():
        raise ValueError("a must be contiguous (row-major M x K)")
    if not (a.is_cuda and b.is_cuda and scale_a.is_cuda and scale_b.is_cuda):
        raise ValueError("all tensors must be on the GPU")
    dev = a.get_device()
    _check_devices(dev, (("b", b), ("scale_a", scale_a), ("scale_b", scale_b), ("bias", bias),
                         ("out", out), ("workspace", workspace)))
    for name, s in (("scale_a", scale_a), ("scale_b", scale_b)):
        if s.dtype != torch.float32 or not s.is_contiguous():
            raise ValueError(f"{name} must be contiguous float32")
    want_a, want_b = (1, 1) if m == PER_TENSOR else (M, N)
    if scale_a.numel() != want_a or scale_b.numel() != want_b:
        raise ValueError(f"{'per-tensor' if m == PER_TENSOR else 'row-wise'} scales need "
                         f"{want_a} and {want_b} elements, got {scale_a.numel()} and {scale_b.numel()}")
    if bias is not None:
        if bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous():
            raise ValueError("bias must be a contiguous bf16 GPU vector of length N")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    elif out.dtype != torch.bfloat16 or out.shape != (M, N) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 M x N tensor")
    L = lib()
    stream = _stream_of(dev)
    # The library launches on the current HIP device: make it a's (calls
    # from that device, the usual case, skip the switch).
    switch = torch.cuda.current_device() != dev
    with torch.cuda.device(dev) if switch else contextlib.nullcontext():
        ws_ptr, ws_bytes = None, 0
        if workspace is not None:
            if not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous GPU tensor")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
        elif splits != 1:
            key = (dev, M, N, K, m, bias is not None, config, splits)
            need = _ws_sizes.get(key)
            if need is None:
                need = int(L.fp8_scaled_mm_workspace_size(M, N, K, m, int(bias is not None),
                                                          int(config), int(splits)))
                if len(_ws_sizes) >= 4096:      # many distinct shapes: start over
                    _ws_sizes.clear()
                _ws_sizes[key] = need
            if need > 0:
                ws = _workspace(a.device, stream, need)
                ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
        st = L.fp8_scaled_mm_typed(
            a.data_ptr(), fa, b.data_ptr(), fb, scale_a.data_ptr(), scale_b.data_ptr(),
            bias.data_ptr() if bias is not None else None, out.data_ptr(),
            M, N, K, m, stream, int(config), int(splits), ws_ptr, ws_bytes)
    if st != OK:
        if st in _ARG_ERRORS:
            raise ValueError(f"fp8_scaled_mm: {status_string(st)} (status {st})")
        raise Fp8MMError(st)
    return out


def fp8_quantize(x: torch.Tensor, mode="rowwise", q: torch.Tensor | None = None,
                 scale: torch.Tensor | None = None, fmt="e4m3fn", workspace=True):
    """(q, scale) = dynamic float8 quantisation of a rows x cols bf16 GPU matrix:
    scale = amax/qmax (one value, or one per row), q = RNE(clamp(x/scale, +-qmax))
    as uint8 codes, with qmax = 448 (fmt 'e4m3fn') or 57344 ('e5m2').  `q` and
    `scale` may be passed to reuse buffers.  workspace=True gives the per-tensor
    mode a per-stream workspace (its one-pass path); False runs the two-pass
    path, which needs none."""
    if mode not in _MODES:
        raise ValueError(f"mode must be 'per_tensor' or 'rowwise', got {mode!r}")
    if fmt not in _FORMATS:
        raise ValueError(f"fmt must be 'e4m3fn' or 'e5m2', got {fmt!r}")
    f = _FORMATS[fmt]
    fn_name = "fp8_quantize_e4m3_ws" if f == E4M3FN else "fp8_quantize_e5m2_ws"
    m = _MODES[mode]
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous 2-D bf16 GPU tensor")
    rows, cols = x.shape
    n_scale = 1 if m == PER_TENSOR else rows
    dev = x.get_device()
    _check_devices(dev, (("q", q), ("scale", scale)))
    if q is None:
        q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    elif q.dtype not in (torch.uint8, torch.float8_e4m3fn if f == E4M3FN else torch.float8_e5m2) \
            or tuple(q.shape) != (rows, cols) or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous uint8 (or float8_{fmt}) rows x cols tensor")
    if scale is None:
        scale = torch.empty(n_scale, dtype=torch.float32, device=x.device)
    elif scale.dtype != torch.float32 or scale.numel() != n_scale or not scale.is_contiguous():
        raise ValueError(f"scale must be a contiguous float32 tensor of {n_scale} elements")
    stream = _stream_of(dev)
    with torch.cuda.device(dev) if torch.cuda.current_device() != dev else contextlib.nullcontext():
        need = int(lib().fp8_quantize_workspace_size(rows, cols, m)) if workspace else 0
        ws = _workspace(x.device, stream, need, "quantize") if need > 0 else None
        st = getattr(lib(), fn_name)(x.data_ptr() if x.numel() else None,
                                     q.data_ptr() if q.numel() else None, scale.data_ptr(),
                                     rows, cols, m, ws.data_ptr() if ws is not None else None,
                                     need, stream)
    if st != Q_OK:
        msg = f"{fn_name}: {lib().fp8_quantize_status_string(st).decode()} (status {st})"
        if st in _Q_ARG_ERRORS:
            raise ValueError(msg)
        raise RuntimeError(msg)
    return q, scale
