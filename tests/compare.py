"""Comparison gates used by the parity tests and the bench's self-check.

bf16 outputs: the distance in units in the last place on the monotone integer
mapping of bf16 bit patterns (+0 and -0 equal) must be <= 1 against the fp32
oracle; an element further off passes only if it is within 1 ulp of the fp64
twin (the arbiter).

fp32 outputs (d_scale / d_shift, LayerNorm statistics): |gpu - o| must be at
most 1e-5 |o| + 2^-24 A, where A is the sum of the absolute values of the
reduced terms (the scale of the rounding error any fp32 summation order can
make); again the fp64 twin arbitrates elements outside the bound.
"""

from __future__ import annotations

import numpy as np

from oracle.fpmath import bf16_ulp_diff

REL_F32 = 1e-5
U24 = 2.0 ** -24


def bf16_gate(gpu_bits, oracle_bits, twin_bits=None, max_ulp: int = 1) -> dict:
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    d = bf16_ulp_diff(gpu_bits, oracle_bits)
    bad = d > max_ulp
    n_out = int(bad.sum())
    if twin_bits is not None and n_out:
        bad &= bf16_ulp_diff(gpu_bits, twin_bits) > max_ulp
    return {
        "n": int(d.size), "max_ulp": int(d.max()) if d.size else 0,
        "n_ulp_gt0": int((d > 0).sum()), "n_outside_oracle": n_out,
        "n_fail": int(bad.sum()),
        "worst_index": (np.unravel_index(int(np.argmax(d)), d.shape) if d.size else None),
    }


def f32_gate(gpu, oracle, A, twin=None, rel: float = REL_F32) -> dict:
    gpu = np.asarray(gpu, np.float64)
    o = np.asarray(oracle, np.float64)
    tol = rel * np.abs(o) + U24 * np.asarray(A, np.float64)
    err = np.abs(gpu - o)
    bad = err > tol
    n_out = int(bad.sum())
    if twin is not None and n_out:
        t = np.asarray(twin, np.float64)
        bad &= np.abs(gpu - t) > rel * np.abs(t) + U24 * np.asarray(A, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        relerr = np.where(o != 0, err / np.abs(o), np.where(err == 0, 0.0, np.inf))
    return {
        "n": int(err.size), "max_abs": float(err.max()) if err.size else 0.0,
        "max_rel": float(relerr.max()) if err.size else 0.0,
        "max_err_over_tol": float((err / np.maximum(tol, 1e-300)).max()) if err.size else 0.0,
        "n_outside_oracle": n_out, "n_fail": int(bad.sum()),
    }


def bytes_equal(a, b) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and a.dtype == b.dtype and a.tobytes() == b.tobytes()
