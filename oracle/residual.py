"""ScaleResidualLayerNormScaleShift at a transformer block's norm sites, written
out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages:
  miles_diffusion pull request 108 ("Fused-norm rounding points"; later text
  "Patches"): LayerNormScaleShift and ScaleResidualLayerNormScaleShift are
  re-patched with the autocast rounding points -- fp32 LayerNorm, (1 + scale)
  rounded once to bf16, fp32 modulation, one bf16 rounding at the next matmul's
  input -- at every *_norm1 / *_norm2 site of the blocks.
  RL-Kernel pull request 538, "Prior art & reuse decision": the fused residual +
  LayerNorm + scale/shift operator of another library (with gated variants),
  hidden width 3072, its modulation taken as chunks of a 6-way modulation.

Reading (the pages give no formula; this is the plainest one the names and the
rounding points support):
  mod [B, 3D] = (shift | scale | gate), the chunk order of one norm site of a
  block's 6-way modulation;
  u   = bf16(gate * x)                  eager bf16 multiply (exact product, one rounding)
  h   = bf16(residual + u)              eager bf16 add: the updated residual stream
  out = bf16((n * bf16(1 + scale)) + shift),  n = LayerNorm(h) in fp32 (as in adaln.py)
Backward from g_out (gradient of out) and g_h (gradient of h from the residual
stream), all bf16:
  dh1 = bf16(rstd * ((gy - alpha) - n * beta)),  gy = g_out * m   (LayerNorm backward)
  dh  = bf16(dh1 + g_h)                 autograd's sum of the two bf16 gradients of h
  d_residual = dh,  dx = bf16(dh * gate)
  d_shift = sum_s g_out,  d_scale = sum_s g_out * n,  d_gate = sum_s dh * x   (fp32)
Every reduction is a sequential Neumaier sum in the fp32 oracle.

Pins: tests/test_oracle_pins.py (P-18 .. P-21).
"""

from __future__ import annotations

import numpy as np

from .adaln import EPS, Arith, _bits, _io, _ln_stats, _normalize, _val


def residual_forward(inp: dict, mode: str = "fp32", eps: float = EPS) -> dict:
    """``inp``: x, residual [B, S, D] and mod [B, 3D] as bf16 bit arrays.
    Returns u, h, mean, rstd, n, m, out (and ``*_bits`` in fp32/fp64 modes)."""
    ar = Arith(mode, _io(inp))
    x = ar.c(_val(inp, "x"))
    res = ar.c(_val(inp, "residual"))
    mod = ar.c(_val(inp, "mod"))
    B, S, D = x.shape
    shift, scale, gate = mod[:, :D], mod[:, D:2 * D], mod[:, 2 * D:]
    u = ar.store(gate[:, None, :] * x)
    h = ar.store(res + u)
    mean, var, rstd = _ln_stats(h.reshape(B * S, D), ar, eps)
    n = _normalize(h.reshape(B * S, D), mean, rstd, ar).reshape(B, S, D)
    m = ar.store(ar.c(1.0) + scale)
    out = ar.store(n * m[:, None, :] + shift[:, None, :])
    r = dict(u=u, h=h, mean=mean.reshape(B, S), rstd=rstd.reshape(B, S), n=n, m=m, out=out,
             gate=gate)
    if mode != "exact":
        r.update(h_bits=_bits(h), out_bits=_bits(out))
    return r


def residual_backward(inp: dict, fwd: dict, mode: str = "fp32", want_abs: bool = False) -> dict:
    """``inp``: g_out, g_h [B, S, D] as bf16 bit arrays (plus the forward's x).
    Returns dh1, dh (= d_residual), dx, d_shift, d_scale, d_gate, d_mod
    (= d_shift | d_scale | d_gate) and, with ``want_abs``, A (sum of |terms|)
    of d_mod."""
    ar = Arith(mode, _io(inp))
    x = ar.c(_val(inp, "x"))
    g = ar.c(_val(inp, "g_out"))
    gh = ar.c(_val(inp, "g_h"))
    B, S, D = g.shape
    R = B * S
    m, n, rstd, gate = fwd["m"], fwd["n"], fwd["rstd"], fwd["gate"]
    gy = g * m[:, None, :]                                            # exact in fp32
    gyT = np.ascontiguousarray(gy.reshape(R, D).T)
    nT = np.ascontiguousarray(n.reshape(R, D).T)
    Dt = ar.c(D)
    alpha = ar.sum(iter(gyT), (R,)) / Dt
    beta = ar.sum((gyT[d] * nT[d] for d in range(D)), (R,)) / Dt
    rs = rstd.reshape(R)[:, None]
    dh1 = ar.store(rs * ((gy.reshape(R, D) - alpha[:, None]) - n.reshape(R, D) * beta[:, None]))
    dh1 = dh1.reshape(B, S, D)
    dh = ar.store(dh1 + gh)
    dx = ar.store(dh * gate[:, None, :])

    r1 = ar.sum((g[:, s, :] for s in range(S)), (B, D), want_abs)
    r2 = ar.sum((g[:, s, :] * n[:, s, :] for s in range(S)), (B, D), want_abs)
    r3 = ar.sum((dh[:, s, :] * x[:, s, :] for s in range(S)), (B, D), want_abs)
    (d_shift, A1), (d_scale, A2), (d_gate, A3) = (r if want_abs else (r, None) for r in (r1, r2, r3))
    d_shift, d_scale, d_gate = ar.f32(d_shift), ar.f32(d_scale), ar.f32(d_gate)
    res = dict(dh1=dh1, dh=dh, d_residual=dh, dx=dx, d_shift=d_shift, d_scale=d_scale, d_gate=d_gate,
               d_mod=np.concatenate([d_shift, d_scale, d_gate], axis=1))
    if mode != "exact":
        res.update(dh_bits=_bits(dh), dx_bits=_bits(dx))
    if want_abs:
        res["A_d_mod"] = np.concatenate([A1, A2, A3], axis=1)
    return res
