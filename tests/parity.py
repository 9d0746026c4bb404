"""Comparison of GPU bf16 outputs with the oracle, under the parity bound

    |gpu - ref| <= 2 * ulp_bf16(|ref|) + 1e-3 * s[m,n] * sum_k |A[m,k]| |B[n,k]|

evaluated in fp64.  ulp_bf16(x) for x > 0 is 2^(max(floor(log2 x), -126) - 7)
(the spacing of bf16 numbers at x; subnormal spacing below 2^-126) and
2^-133 at x = 0.  A NaN reference requires a NaN result, and a NaN result
requires a NaN reference; an infinite reference requires the same infinity,
and an infinite result the same infinite reference.
"""
import numpy as np


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def ulp_bf16(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)
    exp = np.maximum(e.astype(np.int64) - 1, -126)
    u = np.ldexp(1.0, exp - 7)
    return np.where(a == 0, 2.0 ** -133, u)


def compare(gpu_bits, ref):
    """ref: dict from the oracle (bits, s, mag) for the same elements.
    Returns (n_bad, worst_ratio, first_bad_index)."""
    g = bf16_bits_to_f64(gpu_bits)
    r = bf16_bits_to_f64(ref["bits"])
    tol = 2.0 * ulp_bf16(r) + 1e-3 * ref["s"] * ref["mag"]
    rn, gn = np.isnan(r), np.isnan(g)
    ri, gi = np.isinf(r), np.isinf(g)
    with np.errstate(invalid="ignore"):
        err = np.abs(g - r)
        bad = np.where(rn | gn, rn != gn, np.where(ri | gi, r != g, err > tol))
        ratio = np.where(rn | gn | ri | gi, 0.0, err / tol)
    idx = np.argwhere(bad)
    return int(bad.sum()), float(np.max(ratio)) if ratio.size else 0.0, (tuple(idx[0]) if len(idx) else None)
