"""Comparison rules shared by the tests.

The output tolerance reads "within 2 bf16 ulp of the output" per row r
(a GEMM row, an RMSNorm row, or one attention head vector):

    |y - y_ref| <= 2 * ulp_bf16( max(|y_ref|, 2^-8 * max_j |y_ref[r, j]|) )

with ulp_bf16(v) = 2^(floor(log2 |v|) - 7).  Away from cancellation this is
exactly 2 ulp; the row-scale floor covers outputs near zero, where one
unmirrored association (inside a matrix-core or dot instruction) is
amplified by cancellation.  A row that is zero everywhere must match exactly.
GPU-against-GPU comparisons are always bitwise and never use this.
"""
from __future__ import annotations

import math

import numpy as np


def bits_to_f64(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v) -> np.ndarray:
    """Spacing of bf16 numbers in the binade of |v| (normal range)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    out = np.zeros_like(v)
    nz = v > 0
    e = np.floor(np.log2(v[nz]))
    e = np.maximum(e, -126.0)
    out[nz] = np.exp2(e - 7.0)
    return out


def tolerance(ref_rows: np.ndarray, nulp: float = 2.0, floor_rel: float = 2.0 ** -8) -> np.ndarray:
    """Per-element allowed |difference| for a 2-D reference (rows last-axis vectors)."""
    ref = np.asarray(ref_rows, dtype=np.float64)
    rowmax = np.max(np.abs(ref), axis=-1, keepdims=True)
    mag = np.maximum(np.abs(ref), floor_rel * rowmax)
    return nulp * ulp_bf16(mag)


def check_close_bf16(got_bits, ref_bits, nulp: float = 2.0, what: str = ""):
    """Assert bf16 outputs are within the row-floored ulp rule of a reference.

    Returns a small dict of statistics (max ulp distance, elements over the
    unfloored rule) for reporting.
    """
    got = bits_to_f64(got_bits)
    ref = bits_to_f64(ref_bits)
    if got.shape != ref.shape:
        raise AssertionError(f"{what}: shape {got.shape} != {ref.shape}")
    if np.isnan(got).any():
        raise AssertionError(f"{what}: NaN in output")
    ref2 = ref.reshape(-1, ref.shape[-1])
    got2 = got.reshape(-1, got.shape[-1])
    tol = tolerance(ref2, nulp)
    diff = np.abs(got2 - ref2)
    bad = diff > tol
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements outside {nulp} bf16 ulp; first at "
            f"row {i} col {j}: got {got2[i, j]!r} ref {ref2[i, j]!r} tol {tol[i, j]!r}")
    plain = diff > nulp * ulp_bf16(np.abs(ref2))
    ulps = np.where(ref2 != 0, diff / np.maximum(ulp_bf16(np.abs(ref2)), 1e-300), diff > 0)
    return {"max_ulp": float(np.max(ulps, initial=0.0)),
            "over_unfloored": int(plain.sum()),
            "bit_equal_share": float(np.mean(got2 == ref2))}


def bound_vs_exact(y_bits, exact, err_abs):
    """|y - exact| <= err_abs + 1/2 ulp_bf16(|exact| + err_abs): the fp32 error
    bound plus one round-to-nearest narrowing.  Returns the boolean mask of
    elements that break it."""
    y = bits_to_f64(y_bits)
    exact = np.asarray(exact, dtype=np.float64)
    err_abs = np.asarray(err_abs, dtype=np.float64)
    bound = err_abs + 0.5 * ulp_bf16(np.abs(exact) + err_abs)
    # an exact zero with zero error bound must be exactly zero
    return np.abs(y - exact) > bound


def gamma(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32 (u = 2^-24)."""
    u = 2.0 ** -24
    return n * u / (1.0 - n * u)


def gemm_depth(K: int, KB: int = 32, KC: int = 512) -> int:
    """Longest chain of roundings any product sees under the segment schedule:
    inside its block, into its segment, then through the segment fold."""
    S = math.ceil(K / KC)
    return min(K, KB) + min(KC // KB, math.ceil(K / KB)) + S
