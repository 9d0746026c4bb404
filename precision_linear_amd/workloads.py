"""Seeded synthetic inputs for the FP8 scaled matrix multiply.

This module is the only code shared by the GPU path's tests/bench and the CPU
oracle.  It draws random numbers and prepares operand bytes; it holds none of
the multiply's arithmetic (no decoding, no accumulation, no scaling of
products, no output rounding).  Conversions to bf16 and to float8_e4m3fn are
done with torch's CPU casts, exactly as the input recipe of the gist
"matmul_fp8.py" (a-r-r-o-w), functions `get_scale` and `benchmark`, prepares
its operands: amax -> scale = amax / 448 -> x / scale -> clamp to +-448 ->
cast to e4m3fn.  The clamp matters because torch's e4m3fn cast does not
saturate (anything at or above 464 in magnitude becomes NaN).  The gist's
benchmark also takes float8_e5m2 operands; those use 57344 (the e5m2 finfo
maximum) in place of 448 and torch's e5m2 cast.

Layouts produced (all C-contiguous numpy arrays):
  a        uint8  [M, K]   float8 codes (e4m3fn unless the workload says
                           e5m2), K fastest
  b        uint8  [N, K]   float8 codes, K fastest (the "TN" layout: the
                           K x N column-major operand of the pages, stored
                           as its N x K transpose)
  scale_a  float32 [1] (per-tensor) or [M] (row-wise)
  scale_b  float32 [1] (per-tensor) or [N] (row-wise)
  bias     uint16  [N] bf16 bit patterns, or None

Seeds: numpy PCG64 streams keyed by SeedSequence([42, workload_id,
tensor_id, row_block]); 42 is the gist's seed (function `benchmark`).
"""
from __future__ import annotations

import dataclasses
import hashlib
import zlib
from typing import Optional

import numpy as np

PER_TENSOR = 0
ROWWISE = 1
MODE_NAMES = {PER_TENSOR: "per_tensor", ROWWISE: "rowwise"}
E4M3_MAX = 448.0
E5M2_MAX = 57344.0
FORMATS = ("e4m3fn", "e5m2")
BASE_SEED = 42


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    mode: int            # PER_TENSOR or ROWWISE
    recipe: str          # "normal", "skinny", "codes"
    bias: bool = False
    a_format: str = "e4m3fn"
    b_format: str = "e4m3fn"

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def algorithmic_bytes(self) -> int:
        """Bytes the multiply must move at least once: both fp8 operands,
        the fp32 scales, the bf16 bias and the bf16 output."""
        sa = 4 * (self.M if self.mode == ROWWISE else 1)
        sb = 4 * (self.N if self.mode == ROWWISE else 1)
        bias = 2 * self.N if self.bias else 0
        return self.M * self.K + self.N * self.K + sa + sb + bias + 2 * self.M * self.N


def _wl(name, M, N, K, mode, recipe, bias=False, a_format="e4m3fn", b_format="e4m3fn"):
    return Workload(name, M, N, K, mode, recipe, bias, a_format, b_format)


# The synthetic workloads: square shapes with N(0,1) inputs quantised by amax,
# skinny inference shapes (activations N(0,1), weights N(0,0.02), bf16 bias)
# and their one-in-eight column shards,
# ragged shapes whose operands are raw e4m3fn codes, and the gist's mid-size
# shape sweep with N(0,1) inputs.
WORKLOADS = {w.name: w for w in [
    _wl("sq256_pt", 256, 256, 256, PER_TENSOR, "normal"),
    _wl("sq2048_rw", 2048, 2048, 2048, ROWWISE, "normal"),
    _wl("sq8192_pt", 8192, 8192, 8192, PER_TENSOR, "normal"),
    _wl("sq8192_rw", 8192, 8192, 8192, ROWWISE, "normal"),
] + [
    _wl(f"skinny_m{m}_k{k}_n{n}", m, n, k, ROWWISE, "skinny", True)
    for (k, n) in ((8192, 28672), (28672, 8192)) for m in (16, 64, 128)
] + [
    # one GPU's share of the skinny shapes when B (and its scales and bias)
    # is split by output columns over 8 GPUs: N / 8 columns, A replicated
    _wl(f"shard8_m{m}_k{k}_n{n}", m, n, k, ROWWISE, "skinny", True)
    for (k, n) in ((8192, 3584), (28672, 1024)) for m in (16, 64, 128)
] + [
    _wl(f"ragged_{m}x{n}x{k}_{MODE_NAMES[mode]}", m, n, k, mode, "codes")
    for (m, n, k) in ((4096, 4096, 32), (4095, 4097, 96), (8191, 1000, 4160),
                      (16384, 16384, 8192))
    for mode in (PER_TENSOR, ROWWISE)
] + [
    # the gist "matmul_fp8.py" `main` shape sweep (M, K, N), both scaling modes
    _wl(f"gist_m{m}_k{k}_n{n}_{MODE_NAMES[mode]}", m, n, k, mode, "normal")
    for m in (512, 1152, 2304, 4608)
    for (k, n) in ((3072, 12288), (12288, 3072))
    for mode in (PER_TENSOR, ROWWISE)
] + [
    # e5m2 operands (the gist's other float8 dtype), and mixed e4m3fn x e5m2
    _wl(f"fmt_{m}x{n}x{k}_{fa}_{fb}_{MODE_NAMES[mode]}", m, n, k, mode, recipe,
        a_format=fa, b_format=fb)
    for (m, n, k, recipe) in ((2048, 2048, 2048, "normal"), (8192, 8192, 8192, "normal"),
                              (4095, 4097, 96, "codes"))
    for (fa, fb) in (("e5m2", "e5m2"), ("e4m3fn", "e5m2"), ("e5m2", "e4m3fn"))
    for mode in (PER_TENSOR, ROWWISE)
]}


@dataclasses.dataclass
class Inputs:
    a: np.ndarray
    b: np.ndarray
    scale_a: np.ndarray
    scale_b: np.ndarray
    bias: Optional[np.ndarray]
    mode: int
    a_format: str = "e4m3fn"
    b_format: str = "e4m3fn"

    @property
    def shape(self):
        return self.a.shape[0], self.b.shape[0], self.a.shape[1]

    def sha256(self) -> dict:
        out = {}
        for k in ("a", "b", "scale_a", "scale_b", "bias"):
            v = getattr(self, k)
            if v is not None:
                out[k] = hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
        return out


def _rng(workload_key: int, tensor_id: int, block: int = -1) -> np.random.Generator:
    key = [BASE_SEED, workload_key, tensor_id] + ([block] if block >= 0 else [])
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def _blocked(shape, fill, nblk_max=64):
    """Fill a 2-D array in row blocks, each from its own seeded stream (the
    block layout depends on the shape only, so results do not depend on the
    thread count)."""
    from concurrent.futures import ThreadPoolExecutor
    rows = shape[0]
    nblk = max(1, min(nblk_max, rows))
    bounds = [rows * i // nblk for i in range(nblk + 1)]
    out = [None] * nblk

    def job(i):
        out[i] = fill(i, (bounds[i + 1] - bounds[i],) + tuple(shape[1:]))

    with ThreadPoolExecutor(max_workers=min(8, nblk)) as ex:
        list(ex.map(job, range(nblk)))
    return np.ascontiguousarray(np.concatenate(out, axis=0))


def _torch():
    import torch  # local import: torch is only a casting library here
    return torch


def _bf16_normal(key, tensor_id, shape, std=1.0) -> np.ndarray:
    """float32 N(0, std) draws passed through torch's bf16 cast; returned as
    float32 holding bf16-representable values."""
    torch = _torch()
    x = _blocked(shape, lambda i, shp: _rng(key, tensor_id, i).standard_normal(shp, dtype=np.float32))
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()


def _quantise(x: np.ndarray, rowwise: bool, fmt: str = "e4m3fn"):
    """amax/qmax scale (whole tensor or per row of the K-fastest layout),
    then x/scale clamped to +-qmax and cast by torch; qmax = 448 (e4m3fn) or
    57344 (e5m2)."""
    torch = _torch()
    qmax = E4M3_MAX if fmt == "e4m3fn" else E5M2_MAX
    dtype = torch.float8_e4m3fn if fmt == "e4m3fn" else torch.float8_e5m2
    t = torch.from_numpy(x)
    if rowwise:
        amax = t.abs().amax(dim=1)
    else:
        amax = t.abs().amax().reshape(1)
    amax = torch.where(amax > 0, amax, torch.ones_like(amax))
    scale = amax / torch.tensor(qmax, dtype=torch.float32)
    q = (t / (scale[:, None] if rowwise else scale)).clamp(-qmax, qmax)
    codes = q.to(dtype).view(torch.uint8).numpy()
    return np.ascontiguousarray(codes), scale.numpy().astype(np.float32)


# The finite byte codes of each format: e4m3fn has NaN at 0x7F and 0xFF; e5m2
# has infinities and NaNs wherever the exponent field is all ones.
_FINITE_CODES = {
    "e4m3fn": np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8),
    "e5m2": np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8),
}
_NON_NAN_CODES = _FINITE_CODES["e4m3fn"]


def _codes(key, tensor_id, shape, zero_frac=0.01, fmt="e4m3fn") -> np.ndarray:
    pool = _FINITE_CODES[fmt]

    def fill(i, shp):
        rng = _rng(key, tensor_id, i)
        c = pool[rng.integers(0, pool.size, size=shp, dtype=np.int64)]
        c[rng.random(shp, dtype=np.float32) < zero_frac] = 0
        return c
    return _blocked(shape, fill)


def _log_uniform_scales(rng, n) -> np.ndarray:
    return np.exp2(rng.uniform(-8.0, 4.0, size=n)).astype(np.float32)


def make_inputs(M: int, N: int, K: int, mode: int, recipe: str, bias: bool = False,
                key: int = 0, a_format: str = "e4m3fn", b_format: str = "e4m3fn") -> Inputs:
    """Seeded inputs for an (M, N, K) problem.  `key` selects the stream."""
    rowwise = mode == ROWWISE
    if a_format not in FORMATS or b_format not in FORMATS:
        raise ValueError(f"formats must be among {FORMATS}")
    if recipe in ("normal", "skinny"):
        a_f = _bf16_normal(key, 0, (M, K))
        b_f = _bf16_normal(key, 1, (N, K), std=0.02 if recipe == "skinny" else 1.0)
        a, sa = _quantise(a_f, rowwise, a_format)
        b, sb = _quantise(b_f, rowwise, b_format)
        del a_f, b_f
    elif recipe == "codes":
        a = _codes(key, 0, (M, K), fmt=a_format)
        b = _codes(key, 1, (N, K), fmt=b_format)
        sa = _log_uniform_scales(_rng(key, 2), M if rowwise else 1)
        sb = _log_uniform_scales(_rng(key, 3), N if rowwise else 1)
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    bias_bits = None
    if bias:
        bias_bits = _bf16_bits_normal(_rng(key, 4), N)
    return Inputs(a, b, sa, sb, bias_bits, mode, a_format, b_format)


def bf16_matrix_bits(rows: int, cols: int, key: int, std: float = 1.0) -> np.ndarray:
    """Seeded rows x cols matrix of N(0, std) draws cast to bf16 by torch,
    returned as uint16 bit patterns (the quantiser's input)."""
    torch = _torch()
    x = _bf16_normal(key, 5, (rows, cols), std)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _bf16_bits_normal(rng, n) -> np.ndarray:
    torch = _torch()
    x = rng.standard_normal(n, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def workload_key(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def make_workload(name: str) -> Inputs:
    w = WORKLOADS[name]
    return make_inputs(w.M, w.N, w.K, w.mode, w.recipe, w.bias, key=workload_key(name),
                       a_format=w.a_format, b_format=w.b_format)
