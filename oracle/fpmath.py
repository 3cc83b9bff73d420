"""Floating-point building blocks of the oracle (test infrastructure only).

* ``bf16_round``: IEEE round-to-nearest-even to bfloat16, the rounding PyTorch's
  ``.to(torch.bfloat16)`` performs and the one the autocast rounding points of
  miles_diffusion pull request 108 ("Patches": bf16 (1 + scale) rounding) refer
  to.  Works from float32 or float64 with a single rounding.
* ``nsum``: the sequential Neumaier-compensated sum the RL-Kernel pull request
  538 reference uses for its token sums ("What": independent CPU FP32 reference
  with sequential Neumaier token sums).  Pinned against ``math.fsum`` and exact
  rational sums in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------- bfloat16 --
def bits_to_f32(b) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 values, exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _round_f32_bits_to_bf16(u32: np.ndarray) -> np.ndarray:
    u = u32.astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def f32_to_bf16_bits(v) -> np.ndarray:
    """Round float32 values to bfloat16, nearest with ties to even.

    NaN maps to the quiet NaN 0x7FC0 (sign kept); overflow rounds to +-inf.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = _round_f32_bits_to_bf16(v.view(np.uint32))
    nan = np.isnan(v)
    if nan.any():
        out[nan] = (v.view(np.uint32)[nan] >> 16).astype(np.uint16) | 0x7FC0
    return out


def f64_to_bf16_bits(v) -> np.ndarray:
    """Round float64 values to bfloat16 with ONE rounding (nearest, ties to even).

    Goes through float32 with round-to-odd: the float32 value is first taken
    toward zero and its last bit set when it is inexact, so the second
    rounding (float32 -> bfloat16, 16 fewer bits) cannot double-round.
    """
    v = np.ascontiguousarray(v, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        f = v.astype(np.float32)
    bits = f.view(np.uint32).copy()
    f64back = f.astype(np.float64)
    finite = np.isfinite(v) & np.isfinite(f64back)
    away = finite & (np.abs(f64back) > np.abs(v))
    # step one float32 ulp toward zero where the nearest rounding went away
    bits[away] -= 1
    f = bits.view(np.float32)
    inexact = finite & (f.astype(np.float64) != v)
    bits[inexact] |= 1
    out = _round_f32_bits_to_bf16(bits)
    # values whose float32 rounding overflowed: let the float32 path decide
    ovf = np.isfinite(v) & ~np.isfinite(f64back)
    if ovf.any():
        out[ovf] = np.where(v[ovf] > 0, 0x7F80, 0xFF80).astype(np.uint16)
    nan = np.isnan(v)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_round(v) -> np.ndarray:
    """Round to bfloat16 and return the value in the input's float dtype."""
    v = np.asarray(v)
    if v.dtype == np.float64:
        return bits_to_f32(f64_to_bf16_bits(v)).astype(np.float64)
    return bits_to_f32(f32_to_bf16_bits(v))


# ------------------------------------------------------------------ Neumaier --
def nsum_stream(terms, shape, dtype, want_abs: bool = False):
    """Sequential Neumaier sum of the arrays yielded by ``terms`` (ascending order).

    For every element: s = c = +0; for each term x: t = s + x; if |s| >= |x| then
    c += (s - t) + x else c += (x - t) + s; s = t.  The result is s + c.  All
    operations are IEEE operations in ``dtype``.  With ``want_abs`` also returns
    A = sum |x| accumulated in float64 (the error scale the tolerance uses).
    """
    s = np.zeros(shape, dtype)
    c = np.zeros(shape, dtype)
    t = np.empty(shape, dtype)
    e1 = np.empty(shape, dtype)
    e2 = np.empty(shape, dtype)
    big = np.empty(shape, bool)
    A = np.zeros(shape, np.float64) if want_abs else None
    for x in terms:
        x = np.asarray(x, dtype=dtype)
        np.add(s, x, out=t)
        np.greater_equal(np.abs(s), np.abs(x), out=big)
        np.subtract(s, t, out=e1)
        np.add(e1, x, out=e1)
        np.subtract(x, t, out=e2)
        np.add(e2, s, out=e2)
        np.copyto(e2, e1, where=big)
        np.add(c, e2, out=c)
        s, t = t, s
        if want_abs:
            A += np.abs(x).astype(np.float64)
    res = (s + c).astype(dtype)
    return (res, A) if want_abs else res


def nsum(x, axis: int = -1, dtype=np.float32, want_abs: bool = False):
    """Sequential Neumaier sum of ``x`` along ``axis`` in ``dtype``."""
    x = np.asarray(x, dtype=dtype)
    xm = np.moveaxis(x, axis, 0)
    return nsum_stream(iter(xm), xm.shape[1:], dtype, want_abs)


# ----------------------------------------------------------------- ulp tools --
def bf16_ordered(bits) -> np.ndarray:
    """Map bf16 bit patterns to integers that are monotone in value (+0 == -0)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_diff(a_bits, b_bits) -> np.ndarray:
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))
