"""Comparison gates used by the parity tests and the bench's self-check.

bf16 outputs: the distance in units in the last place on the monotone integer
mapping of bf16 bit patterns (+0 and -0 equal) must be <= 1 against the fp32
oracle; an element further off passes only if it is within 1 ulp of the fp64
twin (the arbiter).

bf16 outputs of an fp32-accumulating matrix-core contraction (proj_out): an
element outside both 1-ulp gates still passes when |gpu - e| <= ulp(e) +
kappa 2^-24 A, e the exact sum (the oracle in exact mode), A the sum of the
absolute values of its terms and kappa the number of fp32 roundings along the
longest accumulation path -- the classical bound for recursive summation in
fp32 (Higham, Accuracy and Stability of Numerical Algorithms, ch. 4), plus one
bf16 ulp for the final rounding.  It matters only where the sum cancels.

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


def bf16_ulp_at(v) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (the subnormal spacing below 2^-126)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (np.maximum(e, -126) - 7), 2.0 ** -133)


def bf16_accum_gate(gpu_bits, oracle_bits, twin_bits, exact, A, kappa: int) -> dict:
    """bf16_gate, then the fp32 accumulation bound for the elements it rejects."""
    r = bf16_gate(gpu_bits, oracle_bits, twin_bits)
    gpu_bits = np.asarray(gpu_bits, np.uint16)
    d1 = bf16_ulp_diff(gpu_bits, oracle_bits)
    bad = (d1 > 1) & (bf16_ulp_diff(gpu_bits, twin_bits) > 1)
    g = (gpu_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    e = np.asarray(exact, np.float64)
    tol = bf16_ulp_at(e) + kappa * U24 * np.asarray(A, np.float64)
    within = np.abs(g - e) <= tol
    r["n_outside_ulp_gates"] = int(bad.sum())
    r["n_fail"] = int((bad & ~within).sum())
    r["max_err_over_bound"] = float((np.abs(g - e) / tol).max()) if g.size else 0.0
    return r


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
