"""Forward and backward of the AdaLN final modulation, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source of every step (page titles and sections; the pages print no code):

  RL-Kernel pull request 538, "What":
      scale, shift = (SiLU(temb) @ W^T + b).chunk(2)      3072 -> 6144, scale first
      out = LayerNorm(x, eps=1e-6, no affine) * (1 + scale) + shift
      d_scale, d_shift are token sums accumulated in FP32; the CPU reference
      sums tokens sequentially with Neumaier compensation.
  miles_diffusion pull request 108 ("Fused-norm rounding points"; later text
  "Patches"): LayerNorm computes and returns fp32, (1 + scale) is rounded once
  to bf16, the modulation is fp32, one bf16 rounding at the next consumer.
  RL-Kernel pull request 538, review thread (automated review of the reference
  projection): the SiLU derivative is sigmoid * (1 + z * (1 - sigmoid)); its
  worked value at z = 1 is about 0.9277.  The same thread asks that every
  reduction of the reference be compensated (input gradient and bias gradient
  included), which this oracle does: every sum below is an NSum.

Readings where the pages leave a step open:
  * SiLU is evaluated in float64 and rounded to float32, then to bf16 (its
    output is the bf16 input of the projection matmul).
  * The projection accumulates in fp32, adds the bias in fp32, then rounds
    once to bf16 (emb is a bf16 tensor: scale | shift).
  * LayerNorm: biased variance (divide by D), eps = float32(1e-6) inside the
    square root, two passes (mean, then the mean of squared deviations),
    correctly rounded sqrt and division.
  * The modulation is (n * m) + shift as two fp32 operations (no fused
    multiply-add), m = bf16(1 + scale); the output is rounded once to bf16.
  * Backward: the upstream gradient g is bf16.  gy = g * m (exact);
    alpha = sum(gy)/D, beta = sum(gy * n)/D; dx = bf16(rstd*((gy-alpha)-n*beta)).
    The gradient passes straight through the bf16 rounding of (1 + scale):
    d_scale = sum_s g * n, d_shift = sum_s g, both kept in fp32.
  * Projection backward from the fp32 d_emb: da = sum_j d_emb_j * W_jk,
    dtemb = bf16(da * silu'(z)), dW = bf16(sum_b d_emb_bj * a_bk),
    db = bf16(sum_b d_emb_bj).
  * Every product of the projection, forward and backward, is exact: the
    pages give the projection as a fixed-order GPU kernel accumulating in
    fp32, where a * b + acc is a fused multiply-add (one rounding), and say
    nothing of rounding a product on its own.  In fp32 mode each product
    enters the sum as two fp32 terms whose sum is the product (its fp32
    rounding and the exact remainder); bf16 x bf16 products are exact in
    fp32 anyway, so this changes only the backward's fp32 x bf16 products.

Arithmetic modes:
  "fp32"  the oracle proper: every operation an IEEE float32 operation, every
          reduction a sequential Neumaier sum in float32.
  "fp64"  the fp64 twin (arbiter): the same steps in float64, rounded only at
          the storage points -- a, emb, m, out, dx, dtemb, dW, db to bf16 (one
          rounding each) and the LayerNorm output n, d_scale, d_shift to fp32.
  "exact" float64 with no rounding at all; used for finite-difference checks.

Parity pins live in tests/test_oracle_pins.py; nothing here is unpinned.
"""

from __future__ import annotations

import numpy as np

from .fpmath import (bits_to_f32, bf16_round, f32_to_bf16_bits, f64_to_bf16_bits,
                     nsum_stream)

EPS = 1e-6


class Arith:
    """The arithmetic of one mode: working dtype, storage roundings, sums.

    ``io`` is the storage type of the operator's tensors: "bf16" (the
    autocast rounding points) or "fp32" (the FP32 execution the pages also
    measure: every stored tensor is fp32, so no bf16 rounding anywhere)."""

    def __init__(self, mode: str, io: str = "bf16"):
        if mode not in ("fp32", "fp64", "exact"):
            raise ValueError(mode)
        if io not in ("bf16", "fp32"):
            raise ValueError(io)
        self.mode = mode
        self.io = io
        self.dt = np.float32 if mode == "fp32" else np.float64

    def c(self, v):
        """Cast to the working dtype (exact for every value fed in)."""
        return np.asarray(v, dtype=self.dt)

    def bf16(self, v):
        """Storage rounding to bfloat16 (identity in exact mode)."""
        if self.mode == "exact":
            return np.asarray(v, dtype=np.float64)
        return bf16_round(np.asarray(v, dtype=self.dt))

    def f32(self, v):
        """Storage rounding to float32 (identity in fp32 and exact modes)."""
        if self.mode == "fp64":
            return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)
        return np.asarray(v, dtype=self.dt)

    def store(self, v):
        """Rounding at a storage point: to bf16, or to fp32 for fp32 storage."""
        return self.bf16(v) if self.io == "bf16" else self.f32(v)

    def sum(self, terms, shape, want_abs=False):
        return nsum_stream(terms, shape, self.dt, want_abs)

    def prod(self, x, y):
        """The terms of the exact products x * y (fp32 or bf16 operands).

        float64 holds such a product exactly (at most 48 significant bits), so
        the fp64 and exact modes yield it as one term.  In fp32 mode it is
        yielded as hi = fp32(p) and lo = p - hi, both exact in fp32 (lo has
        at most 24 significant bits) unless |p| is below about 2^-100."""
        p = np.asarray(x, np.float64) * np.asarray(y, np.float64)
        if self.mode != "fp32":
            return (p,)
        hi = p.astype(np.float32)
        return (hi, (p - hi.astype(np.float64)).astype(np.float32))


def _silu64(z):
    return z / (1.0 + np.exp(-z))


def _dsilu64(z):
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def _val(inp: dict, key: str) -> np.ndarray:
    """Input values: ``inp[key + '_val']`` (float64, exact mode), fp32 values
    (fp32 storage) or the bf16 bits."""
    if key + "_val" in inp:
        return np.asarray(inp[key + "_val"], dtype=np.float64)
    v = np.asarray(inp[key])
    if v.dtype == np.float32:
        return v
    return bits_to_f32(v)


def _io(inp: dict) -> str:
    return inp.get("io", "bf16")


def silu_act(temb, ar: Arith):
    """a = SiLU(temb) at its storage rounding (bf16, or fp32); SiLU in float64,
    rounded to float32 in fp32 mode."""
    z = np.asarray(temb).astype(np.float64)
    v = _silu64(z)
    if ar.mode == "fp32":
        v = v.astype(np.float32)
    return ar.store(v)


def dsilu(temb, ar: Arith):
    """silu'(z) = sigma * (1 + z * (1 - sigma)) in float64 (float32 result in fp32 mode)."""
    z = np.asarray(temb).astype(np.float64)
    v = _dsilu64(z)
    return ar.c(v.astype(np.float32)) if ar.mode == "fp32" else v


def projection(a, W, bias, ar: Arith, want_abs=False):
    """emb[b, j] = bf16(sum_k a[b,k] * W[j,k] + bias[j])  (scale = emb[:, :D])."""
    WT = np.ascontiguousarray(ar.c(W).T)                             # [K, N]
    bias = ar.c(bias)
    a = ar.c(a)
    B, K = a.shape
    N = WT.shape[1]
    terms = (t for k in range(K) for t in ar.prod(a[:, k:k + 1], WT[k][None, :]))
    r = ar.sum(terms, (B, N), want_abs)
    acc, A = (r if want_abs else (r, None))
    emb = ar.store(acc + bias)
    return (emb, A) if want_abs else emb


def _ln_stats(x2, ar: Arith, eps: float = EPS):
    """Per-row mean, biased variance and rstd of x2 [R, D] (two passes)."""
    R, D = x2.shape
    xT = np.ascontiguousarray(x2.T)                                   # [D, R]
    Dt = ar.c(D)
    mean = ar.sum(iter(xT), (R,)) / Dt
    dT = xT - mean[None, :]
    var = ar.sum((dT[d] * dT[d] for d in range(D)), (R,)) / Dt
    eps_t = ar.c(np.float32(eps))
    rstd = ar.c(1.0) / np.sqrt(var + eps_t)
    return mean, var, rstd


def _normalize(x2, mean, rstd, ar: Arith):
    """n = (x - mean) * rstd, stored as the fp32 LayerNorm output."""
    return ar.f32((x2 - mean[:, None]) * rstd[:, None])


def forward(inp: dict, mode: str = "fp32", eps: float = EPS, want_abs: bool = False):
    """Forward pass.  ``inp`` holds x, temb, W, bias as bf16 bit arrays, or as
    fp32 arrays with ``inp['io'] == 'fp32'`` (fp32 storage).

    Returns a dict: a, emb, m, mean, rstd, n, out (values in the mode's dtype;
    bf16 quantities hold bf16-representable values) and, for bf16 storage,
    ``*_bits`` uint16 arrays.
    """
    ar = Arith(mode, _io(inp))
    x = ar.c(_val(inp, "x"))
    B, S, D = x.shape
    a = silu_act(_val(inp, "temb"), ar)
    pr = projection(a, _val(inp, "W"), _val(inp, "bias"), ar, want_abs)
    emb, A_emb = pr if want_abs else (pr, None)
    scale, shift = emb[:, :D], emb[:, D:]
    one = ar.c(1.0)
    m = ar.store(one + scale)

    mean, var, rstd = _ln_stats(x.reshape(B * S, D), ar, eps)
    n = _normalize(x.reshape(B * S, D), mean, rstd, ar).reshape(B, S, D)
    out = ar.store(n * m[:, None, :] + shift[:, None, :])
    res = dict(a=a, emb=emb, m=m, mean=mean.reshape(B, S), rstd=rstd.reshape(B, S),
               n=n, out=out, var=var.reshape(B, S))
    if mode != "exact" and ar.io == "bf16":
        res["out_bits"] = _bits(out)
        res["emb_bits"] = _bits(emb)
        res["a_bits"] = _bits(a)
    if want_abs:
        res["A_emb"] = A_emb
    return res


def backward(inp: dict, fwd: dict, mode: str = "fp32", want_abs: bool = False,
             g=None):
    """Backward pass from the upstream gradient ``inp['g']`` (bf16 bits).

    Returns dx, d_scale, d_shift, d_emb (= d_scale | d_shift), da, dtemb, dW, db
    and, for bf16 outputs, ``*_bits``.  With ``want_abs`` also the error scales
    A (sum of |terms|, float64) of d_emb, alpha/beta, da, dW and db.
    """
    ar = Arith(mode, _io(inp))
    g = ar.c(_val(inp, "g") if g is None else g)
    B, S, D = g.shape
    R = B * S
    m, n, rstd = fwd["m"], fwd["n"], fwd["rstd"]
    gy = g * m[:, None, :]                                            # exact in fp32
    gyT = np.ascontiguousarray(gy.reshape(R, D).T)
    nT = np.ascontiguousarray(n.reshape(R, D).T)
    Dt = ar.c(D)
    alpha = ar.sum(iter(gyT), (R,)) / Dt
    beta = ar.sum((gyT[d] * nT[d] for d in range(D)), (R,)) / Dt
    rs = rstd.reshape(R)[:, None]
    dx = ar.store(rs * ((gy.reshape(R, D) - alpha[:, None]) - n.reshape(R, D) * beta[:, None]))
    dx = dx.reshape(B, S, D)

    # token sums over s, per sample
    r1 = ar.sum((g[:, s, :] for s in range(S)), (B, D), want_abs)
    r2 = ar.sum((g[:, s, :] * n[:, s, :] for s in range(S)), (B, D), want_abs)
    d_shift, A_shift = r1 if want_abs else (r1, None)
    d_scale, A_scale = r2 if want_abs else (r2, None)
    d_shift = ar.f32(d_shift)
    d_scale = ar.f32(d_scale)
    d_emb = np.concatenate([d_scale, d_shift], axis=1)                 # [B, 2D]

    W = ar.c(_val(inp, "W"))                                           # [N, K]
    pb = proj_backward(d_emb, fwd["a"], W, _val(inp, "temb"), ar, want_abs)
    da, dtemb, dW_acc, dW, db_acc, db = (pb[k] for k in ("da", "dtemb", "dW_acc", "dW", "db_acc", "db"))
    A_da, A_dW, A_db = pb.get("A_da"), pb.get("A_dW"), pb.get("A_db")

    res = dict(dx=dx, d_scale=d_scale, d_shift=d_shift, d_emb=d_emb, da=da,
               dtemb=dtemb, dW=dW, db=db, dW_acc=dW_acc, db_acc=db_acc,
               alpha=alpha.reshape(B, S), beta=beta.reshape(B, S))
    if mode != "exact" and ar.io == "bf16":
        for k in ("dx", "dtemb", "dW", "db"):
            res[k + "_bits"] = _bits(res[k])
    if want_abs:
        res["A_d_emb"] = np.concatenate([A_scale, A_shift], axis=1)
        res.update(A_da=A_da, A_dW=A_dW, A_db=A_db)
    return res


def proj_backward(d_emb, a, W, temb, ar: Arith, want_abs: bool = False) -> dict:
    """Projection backward from d_emb [B, N] (fp32 values), a [B, K] (bf16
    values), W [N, K] and temb [B, K]: da, dtemb = bf16(da * silu'(temb)),
    dW = bf16(sum_b d_emb_b x a_b), db = bf16(sum_b d_emb_b), every product exact.
    dtemb_acc, dW_acc, db_acc are the values before their single storage
    rounding."""
    d_emb, a, W = ar.c(d_emb), ar.c(a), ar.c(W)
    B, N = d_emb.shape
    K = W.shape[1]
    r3 = ar.sum((t for j in range(N) for t in ar.prod(d_emb[:, j:j + 1], W[j][None, :])), (B, K), want_abs)
    da, A_da = r3 if want_abs else (r3, None)
    dtemb_acc = da * dsilu(temb, ar)          # the value dtemb rounds once to storage
    dtemb = ar.store(dtemb_acc)
    r4 = ar.sum((t for b in range(B) for t in ar.prod(d_emb[b][:, None], a[b][None, :])), (N, K), want_abs)
    dW_acc, A_dW = r4 if want_abs else (r4, None)
    r5 = ar.sum((d_emb[b] for b in range(B)), (N,), want_abs)
    db_acc, A_db = r5 if want_abs else (r5, None)
    res = dict(da=da, dtemb=dtemb, dtemb_acc=dtemb_acc, dW_acc=dW_acc, dW=ar.store(dW_acc), db_acc=db_acc,
               db=ar.store(db_acc))
    if want_abs:
        res.update(A_da=A_da, A_dW=A_dW, A_db=A_db)
    return res


def _bits(v):
    v = np.asarray(v)
    if v.dtype == np.float64:
        return f64_to_bf16_bits(v)
    return f32_to_bf16_bits(v)


def sgld_forward_out(inp: dict, fwd: dict):
    """The rollout-side semantics the miles_diffusion pull request 108 summary
    names as wrong: the LayerNorm output is rounded to bf16 and the modulation
    runs in bf16 eager ops (each op rounds to bf16).  Used only as a negative
    control: it must differ from ``forward``'s output."""
    n16 = bf16_round(np.asarray(fwd["n"], dtype=np.float32))
    m = np.asarray(fwd["m"], dtype=np.float32)
    D = m.shape[1]
    shift = np.asarray(fwd["emb"], dtype=np.float32)[:, D:]
    prod = bf16_round(n16 * m[:, None, :])
    return bf16_round(prod + shift[:, None, :])


# ------------------------------------------------------- sampled evaluation --
# For batches too large to run whole, the same steps evaluated for a subset of
# outputs.  Every value goes through the functions above.

def ln_stats(inp: dict, mode: str = "fp32", eps: float = EPS):
    """mean, rstd [B, S] of every row (the saved LayerNorm state)."""
    ar = Arith(mode, _io(inp))
    x = ar.c(_val(inp, "x"))
    B, S, D = x.shape
    mean, _, rstd = _ln_stats(x.reshape(B * S, D), ar, eps)
    return mean.reshape(B, S), rstd.reshape(B, S)


def d_emb_columns(inp: dict, cols, mode: str = "fp32", eps: float = EPS, stats=None):
    """d_emb[:, cols] (d_scale for cols < D, d_shift for cols >= D), every sample."""
    ar = Arith(mode, _io(inp))
    x = ar.c(_val(inp, "x"))
    g = ar.c(_val(inp, "g"))
    B, S, D = x.shape
    mean, rstd = stats if stats is not None else ln_stats(inp, mode, eps)
    cols = np.asarray(cols)
    dcol = np.where(cols < D, cols, cols - D)
    xs = x[:, :, dcol]                                                # [B, S, C]
    gs = g[:, :, dcol]
    n = _normalize(xs.reshape(B * S, -1), mean.reshape(-1), rstd.reshape(-1), ar).reshape(xs.shape)
    terms = np.where((cols < D)[None, None, :], gs * n, gs)
    out = ar.sum((terms[:, s, :] for s in range(S)), (B, len(cols)))
    return ar.f32(out)


def param_grads_rows(inp: dict, rows, mode: str = "fp32", eps: float = EPS, stats=None):
    """dW[rows, :] and db[rows] over the whole batch (bf16 bits, or fp32
    values for fp32 storage)."""
    ar = Arith(mode, _io(inp))
    a = silu_act(_val(inp, "temb"), ar)                               # [B, K]
    de = d_emb_columns(inp, rows, mode, eps, stats)                   # [B, R]
    B = a.shape[0]
    dW = ar.store(ar.sum((t for b in range(B) for t in ar.prod(de[b][:, None], a[b][None, :])),
                         (len(rows), a.shape[1])))
    db = ar.store(ar.sum((de[b] for b in range(B)), (len(rows),)))
    if ar.io == "fp32":
        return dW, db, de
    return _bits(dW), _bits(db), de
