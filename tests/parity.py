"""Comparison rules shared by the parity tests.

GEMM outputs: the method accumulates in fp32 and only the order of the
accumulation differs between the oracle and the GPU.  A literal per-element
relative bound of 1e-3 fails on outputs that cancel to near zero, so the
bound is floored by the size of the terms:

    t = 1e-3 * max(|Y32|, P / sqrt(K)),   P = sum_k |a_hat * b_hat|

fp32 output:  |y - Y32| <= t
bf16 output:  bf16_rne(Y32 - t) <= y <= bf16_rne(Y32 + t)

so that the bf16 output rounding (up to 2^-9 relative) is bracketed rather
than charged against the 1e-3 budget.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_TOL = 1e-3


def gemm_bound(y32: np.ndarray, p: np.ndarray, K: int) -> np.ndarray:
    return REL_TOL * np.maximum(np.abs(y32.astype(np.float64)), p / np.sqrt(K))


def check_gemm(y: np.ndarray, y32: np.ndarray, p: np.ndarray, K: int, out_dtype: str):
    """Return (ok_mask, report dict).  y is fp32 values or bf16 bit patterns."""
    t = gemm_bound(y32, p, K)
    ref = y32.astype(np.float64)
    if out_dtype == "f32":
        yv = y.astype(np.float64)
        ok = np.abs(yv - ref) <= t
    else:
        yv = oracle.bf16_bits_to_f32(y).astype(np.float64)
        lo = oracle.bf16_bits_to_f32(oracle.f32_to_bf16((ref - t).astype(np.float32)))
        hi = oracle.bf16_bits_to_f32(oracle.f32_to_bf16((ref + t).astype(np.float32)))
        ok = (yv >= lo) & (yv <= hi)
    err = np.abs(yv - ref) / np.maximum(np.maximum(np.abs(ref), p / np.sqrt(K)), 1e-30)
    nrm = float(np.linalg.norm(yv - ref) / max(np.linalg.norm(ref), 1e-30))
    return ok, {"max_floored_rel": float(err.max()) if err.size else 0.0,
                "normwise_rel": nrm, "n_bad": int((~ok).sum()), "n": int(ok.size)}


def assert_gemm(y, y32, p, K, out_dtype, what=""):
    ok, rep = check_gemm(y, y32, p, K, out_dtype)
    if not ok.all():
        bad = np.argwhere(~ok.reshape(-1))[:5].ravel()
        raise AssertionError(f"{what}: {rep}; first bad flat indices {bad.tolist()}")
    return rep
