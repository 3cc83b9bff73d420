"""The output projection after the final modulation (proj_out, 3072 -> 64),
written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages:
  RL-Kernel pull request 538, "What" and "Scope / Known limitations": the later
  3072 -> 64 proj_out belongs to another operator (latent_proj_gemm) and is not
  part of the final modulation's.
  miles_diffusion pull request 108, "Fused-norm rounding points": under
  autocast the modulated output stays fp32 and its single bf16 rounding happens
  at the input of the next matmul -- this projection.

Reading (the pages name the operator and its width, not its arithmetic; this is
the plainest one, the autocast Linear with the final modulation's projection
arithmetic):
  latent[t, o] = bf16(fl32(sum_k out[t, k] * Wp[o, k]) + bp[o])    out bf16 [T, 3072]
every product exact, the sum in fp32, the bias added in fp32, one bf16
rounding; T = B * S tokens, each token on its own.  Backward from the bf16
gradient d_lat [T, 64]:
  d_out[t, k] = bf16(fl32(sum_o d_lat[t, o] * Wp[o, k]))
  dWp[o, k]   = bf16(fl32(sum_t d_lat[t, o] * out[t, k]))
  dbp[o]      = bf16(fl32(sum_t d_lat[t, o]))
Every reduction is a sequential Neumaier sum in the fp32 oracle.

Pins: tests/test_oracle_pins.py (P-24, P-25).
"""

from __future__ import annotations

import numpy as np

from .adaln import Arith, _bits, _val


def _tokens(v: np.ndarray) -> np.ndarray:
    """[B, S, K] or [T, K] -> [T, K]."""
    return v.reshape(-1, v.shape[-1])


def proj_out_forward(inp: dict, mode: str = "fp32", want_abs: bool = False) -> dict:
    """``inp``: out [T, K] (or [B, S, K]), W [O, K], bias [O] as bf16 bit arrays.
    Returns latent [T, O] (and latent_bits; A_latent with ``want_abs``)."""
    ar = Arith(mode)
    x = ar.c(_tokens(_val(inp, "out")))
    WT = np.ascontiguousarray(ar.c(_val(inp, "W")).T)                 # [K, O]
    bias = ar.c(_val(inp, "bias"))
    T, K = x.shape
    O = WT.shape[1]
    terms = (t for k in range(K) for t in ar.prod(x[:, k:k + 1], WT[k][None, :]))
    r = ar.sum(terms, (T, O), want_abs)
    acc, A = r if want_abs else (r, None)
    latent = ar.store(acc + bias)
    res = dict(latent=latent)
    if mode != "exact":
        res["latent_bits"] = _bits(latent)
    if want_abs:
        res["A_latent"] = A
    return res


def proj_out_backward(inp: dict, mode: str = "fp32", want_abs: bool = False,
                      outputs=("d_out", "dW", "db")) -> dict:
    """``inp``: d_lat [T, O] (or [B, S, O]) bf16 bits, plus the forward's out and W.
    Returns the requested ``outputs`` among d_out [T, K], dW [O, K], db [O]
    (``*_bits``; A_* with ``want_abs``)."""
    ar = Arith(mode)
    x = ar.c(_tokens(_val(inp, "out")))
    W = ar.c(_val(inp, "W"))
    d = ar.c(_tokens(_val(inp, "d_lat")))
    T, K = x.shape
    O = W.shape[0]
    sums = {
        "d_out": lambda: ar.sum((t for o in range(O) for t in ar.prod(d[:, o:o + 1], W[o][None, :])), (T, K),
                                want_abs),
        "dW": lambda: ar.sum((t for i in range(T) for t in ar.prod(d[i][:, None], x[i][None, :])), (O, K), want_abs),
        "db": lambda: ar.sum((d[i] for i in range(T)), (O,), want_abs),
    }
    res = {}
    for k in outputs:
        r = sums[k]()
        v, A = r if want_abs else (r, None)
        res[k] = ar.store(v)
        if mode != "exact":
            res[k + "_bits"] = _bits(res[k])
        if want_abs:
            res["A_" + k] = A
    return res
