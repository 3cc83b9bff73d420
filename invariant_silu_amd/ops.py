"""PyTorch-facing wrappers of the C ABI (include/adaln.h).

PyTorch supplies device memory and the current HIP stream; every computation
runs in the library's kernels.  Tensors are made contiguous, and any tensor
whose data pointer is not 16-byte aligned is copied to an aligned buffer
(``.contiguous()`` alone does not realign a view with a storage offset --
RL-Kernel pull request 538, review thread on misaligned views).
"""

from __future__ import annotations

import torch

from . import lib as _lib

D = 3072
N = 2 * D
EPS = 1e-6


def aligned(t: torch.Tensor) -> torch.Tensor:
    """Contiguous tensor whose data pointer is 16-byte aligned (copies if needed)."""
    t = t.contiguous()
    if t.data_ptr() % 16 != 0:
        out = torch.empty(t.shape, dtype=t.dtype, device=t.device)
        out.copy_(t)
        t = out
    return t


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _shape(t: torch.Tensor, shape, name: str) -> None:
    """The C ABI sees pointers only, so every extent it assumes is checked here,
    before anything reaches it."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rank(t: torch.Tensor, n: int, name: str) -> None:
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")


def _proj_width(W: torch.Tensor, widths=(N, 6 * D)) -> int:
    _rank(W, 2, "W")
    if W.shape[0] not in widths or W.shape[1] != D:
        raise ValueError(f"W must have shape (N, {D}) with N in {widths}, got {tuple(W.shape)}")
    return W.shape[0]


def _rows(x: torch.Tensor, name: str = "x"):
    """(B, S) of a [B, S, 3072] activation."""
    _rank(x, 3, name)
    if x.shape[2] != D:
        raise ValueError(f"{name} must have shape (B, S, {D}), got {tuple(x.shape)}")
    return x.shape[0], x.shape[1]


def _check(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the HIP library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _call(tensors, name: str, *args) -> None:
    """Call entry point `name` with every tensor it receives on one device, that
    device current (the library launches on the current device and checks its
    architecture there)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"{name}: all tensors must be on one GPU, got {sorted(str(d) for d in devs)}")
    with torch.cuda.device(devs.pop()):
        _lib.call(name, *args)


def _ws(op: int, B: int, S: int, H: int, device) -> torch.Tensor:
    n = _lib.workspace_bytes(op, B, S, H)
    if n == 0:
        raise ValueError(f"unsupported sizes for op {op}: B={B} S={S} H={H}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def proj_fwd(temb: torch.Tensor, W: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    """emb [B, N] bf16 = bf16(SiLU(temb) W^T + b), N = W.shape[0]: 6144 for the
    final modulation (scale | shift), 18432 for a block's 6-way modulation
    (shift1 | scale1 | gate1 | shift2 | scale2 | gate2)."""
    Nw = _proj_width(W)
    _rank(temb, 2, "temb")
    _shape(temb, (temb.shape[0], D), "temb")
    _shape(bias, (Nw,), "bias")
    for t, n in ((temb, "temb"), (W, "W"), (bias, "bias")):
        _check(t, torch.bfloat16, n)
    temb, W, bias = aligned(temb), aligned(W), aligned(bias)
    B = temb.shape[0]
    emb = torch.empty((B, W.shape[0]), dtype=torch.bfloat16, device=temb.device)
    ws = _ws(_lib.OP_PROJ_FWD, B, 1, temb.shape[1], temb.device)
    _call((temb, W, bias, emb, ws), "adaln_proj_fwd", temb.data_ptr(), W.data_ptr(), bias.data_ptr(), emb.data_ptr(),
          ws.data_ptr(), ws.numel(), B, temb.shape[1], W.shape[0], _stream(temb.device))
    return emb


def norm_mod_fwd(x: torch.Tensor, emb: torch.Tensor, eps: float = EPS):
    """(out bf16 [B,S,D], mean fp32 [B,S], rstd fp32 [B,S])."""
    B, S = _rows(x)
    _shape(emb, (B, N), "emb")
    _check(x, torch.bfloat16, "x")
    _check(emb, torch.bfloat16, "emb")
    x, emb = aligned(x), aligned(emb)
    B, S, Dx = x.shape
    out = torch.empty_like(x)
    mean = torch.empty((B, S), dtype=torch.float32, device=x.device)
    rstd = torch.empty((B, S), dtype=torch.float32, device=x.device)
    _call((x, emb, out, mean, rstd), "adaln_norm_mod_fwd", x.data_ptr(), emb.data_ptr(), out.data_ptr(),
          mean.data_ptr(), rstd.data_ptr(), B, S, Dx, float(eps), _stream(x.device))
    return out, mean, rstd


def norm_mod_bwd(g: torch.Tensor, x: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor,
                 emb: torch.Tensor):
    """(dx bf16 [B,S,D], d_emb fp32 [B, 2D] = (d_scale | d_shift))."""
    B, S = _rows(x)
    _shape(g, x.shape, "g")
    _shape(mean, (B, S), "mean")
    _shape(rstd, (B, S), "rstd")
    _shape(emb, (B, N), "emb")
    _check(g, torch.bfloat16, "g")
    _check(x, torch.bfloat16, "x")
    _check(mean, torch.float32, "mean")
    _check(rstd, torch.float32, "rstd")
    _check(emb, torch.bfloat16, "emb")
    g, x, mean, rstd, emb = (aligned(t) for t in (g, x, mean, rstd, emb))
    B, S, Dx = x.shape
    dx = torch.empty_like(x)
    d_emb = torch.empty((B, N), dtype=torch.float32, device=x.device)
    ws = _ws(_lib.OP_NORM_MOD_BWD, B, S, Dx, x.device)
    _call((g, x, mean, rstd, emb, dx, d_emb, ws), "adaln_norm_mod_bwd", g.data_ptr(), x.data_ptr(), mean.data_ptr(),
          rstd.data_ptr(), emb.data_ptr(), dx.data_ptr(), d_emb.data_ptr(), ws.data_ptr(), ws.numel(), B, S, Dx,
          _stream(x.device))
    return dx, d_emb


def proj_bwd(d_emb: torch.Tensor, temb: torch.Tensor, W: torch.Tensor, want_f32: bool = False):
    """(dW bf16 [N, 3072], db bf16 [N], dtemb bf16 [B, 3072]); N = W.shape[0]
    (6144 or 18432, as for proj_fwd).  want_f32: also the fp32 values those
    are rounded from, (dW, db, dtemb, dW_f32, db_f32, dtemb_f32)
    (adaln_proj_bwd_acc)."""
    Nw = _proj_width(W)
    _rank(temb, 2, "temb")
    _shape(temb, (temb.shape[0], D), "temb")
    _shape(d_emb, (temb.shape[0], Nw), "d_emb")
    _check(d_emb, torch.float32, "d_emb")
    _check(temb, torch.bfloat16, "temb")
    _check(W, torch.bfloat16, "W")
    d_emb, temb, W = aligned(d_emb), aligned(temb), aligned(W)
    B = temb.shape[0]
    dW = torch.empty_like(W)
    db = torch.empty((W.shape[0],), dtype=torch.bfloat16, device=W.device)
    dtemb = torch.empty_like(temb)
    ws = _ws(_lib.OP_PROJ_BWD, B, 1, D, W.device)
    if not want_f32:
        _call((d_emb, temb, W, dW, db, dtemb, ws), "adaln_proj_bwd", d_emb.data_ptr(), temb.data_ptr(), W.data_ptr(),
              dW.data_ptr(), db.data_ptr(), dtemb.data_ptr(), ws.data_ptr(), ws.numel(), B, temb.shape[1], W.shape[0],
              _stream(W.device))
        return dW, db, dtemb
    dW32 = torch.empty(W.shape, dtype=torch.float32, device=W.device)
    db32 = torch.empty((W.shape[0],), dtype=torch.float32, device=W.device)
    dtemb32 = torch.empty(temb.shape, dtype=torch.float32, device=W.device)
    _call((d_emb, temb, W, dW, db, dtemb, dW32, db32, dtemb32, ws), "adaln_proj_bwd_acc", d_emb.data_ptr(),
          temb.data_ptr(), W.data_ptr(), dW.data_ptr(), db.data_ptr(), dtemb.data_ptr(), dW32.data_ptr(),
          db32.data_ptr(), dtemb32.data_ptr(), ws.data_ptr(), ws.numel(), B, temb.shape[1], W.shape[0],
          _stream(W.device))
    return dW, db, dtemb, dW32, db32, dtemb32


def token_tree_sum(x: torch.Tensor) -> torch.Tensor:
    """Compensated 32-token tree sum over dim 1 of an fp32 [B, S, H] tensor."""
    _rank(x, 3, "x")
    _check(x, torch.float32, "x")
    x = aligned(x)
    B, S, H = x.shape
    out = torch.empty((B, H), dtype=torch.float32, device=x.device)
    ws = _ws(_lib.OP_TOKEN_TREE_SUM, B, S, H, x.device)
    _call((x, out, ws), "token_tree_sum", x.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(), B, S, H,
          _stream(x.device))
    return out


_STORAGE = (torch.bfloat16, torch.float32)


def fwd(x: torch.Tensor, temb: torch.Tensor, W: torch.Tensor, bias: torch.Tensor, eps: float = EPS):
    """One-call forward (adaln_fwd, or adaln_fwd_f32 for fp32 tensors):
    (out, emb, mean, rstd); with bf16 tensors the same bits as proj_fwd
    followed by norm_mod_fwd."""
    B, S = _rows(x)
    _shape(temb, (B, D), "temb")
    _proj_width(W, (N,))
    _shape(bias, (N,), "bias")
    dt = x.dtype
    if dt not in _STORAGE:
        raise TypeError(f"x must be bfloat16 or float32, got {dt}")
    for t, n in ((x, "x"), (temb, "temb"), (W, "W"), (bias, "bias")):
        _check(t, dt, n)
    x, temb, W, bias = aligned(x), aligned(temb), aligned(W), aligned(bias)
    B, S, Dx = x.shape
    emb = torch.empty((B, N), dtype=dt, device=x.device)
    out = torch.empty_like(x)
    mean = torch.empty((B, S), dtype=torch.float32, device=x.device)
    rstd = torch.empty((B, S), dtype=torch.float32, device=x.device)
    _call((temb, W, bias, x, emb, out, mean, rstd), "adaln_fwd" if dt == torch.bfloat16 else "adaln_fwd_f32",
          temb.data_ptr(), W.data_ptr(), bias.data_ptr(), x.data_ptr(), emb.data_ptr(), out.data_ptr(),
          mean.data_ptr(), rstd.data_ptr(), B, S, Dx, float(eps), _stream(x.device))
    return out, emb, mean, rstd


def bwd(g: torch.Tensor, x: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor, emb: torch.Tensor,
        temb: torch.Tensor, W: torch.Tensor):
    """One-call backward (adaln_bwd, or adaln_bwd_f32 for fp32 tensors):
    (dx, d_emb, dW, db, dtemb); with bf16 tensors the same bits as
    norm_mod_bwd followed by proj_bwd."""
    B, S = _rows(x)
    _shape(g, x.shape, "g")
    _shape(mean, (B, S), "mean")
    _shape(rstd, (B, S), "rstd")
    _shape(emb, (B, N), "emb")
    _shape(temb, (B, D), "temb")
    _proj_width(W, (N,))
    dt = x.dtype
    if dt not in _STORAGE:
        raise TypeError(f"x must be bfloat16 or float32, got {dt}")
    for t, n, tdt in ((g, "g", dt), (x, "x", dt), (mean, "mean", torch.float32),
                      (rstd, "rstd", torch.float32), (emb, "emb", dt), (temb, "temb", dt), (W, "W", dt)):
        _check(t, tdt, n)
    g, x, mean, rstd, emb, temb, W = (aligned(t) for t in (g, x, mean, rstd, emb, temb, W))
    B, S, Dx = x.shape
    dx = torch.empty_like(x)
    d_emb = torch.empty((B, N), dtype=torch.float32, device=x.device)
    dW = torch.empty_like(W)
    db = torch.empty((W.shape[0],), dtype=dt, device=W.device)
    dtemb = torch.empty_like(temb)
    f32 = dt == torch.float32
    ws = _ws(_lib.OP_BWD_F32 if f32 else _lib.OP_BWD, B, S, Dx, x.device)
    _call((g, x, mean, rstd, emb, temb, W, dx, d_emb, dW, db, dtemb, ws), "adaln_bwd_f32" if f32 else "adaln_bwd",
          g.data_ptr(), x.data_ptr(), mean.data_ptr(), rstd.data_ptr(), emb.data_ptr(), temb.data_ptr(), W.data_ptr(),
          dx.data_ptr(), d_emb.data_ptr(), dW.data_ptr(), db.data_ptr(), dtemb.data_ptr(), ws.data_ptr(), ws.numel(),
          B, S, Dx, _stream(x.device))
    return dx, d_emb, dW, db, dtemb


def residual_fwd(x: torch.Tensor, residual: torch.Tensor, mod: torch.Tensor, eps: float = EPS):
    """Residual norm site (adaln_residual_fwd): (out, h, mean, rstd) with
    h = bf16(residual + bf16(gate * x)), out = bf16(LN(h) * bf16(1 + scale) + shift),
    mod [B, 3 * 3072] = (shift | scale | gate); bf16 tensors."""
    B, S = _rows(x)
    _shape(residual, x.shape, "residual")
    _shape(mod, (B, 3 * D), "mod")
    for t, n in ((x, "x"), (residual, "residual"), (mod, "mod")):
        _check(t, torch.bfloat16, n)
    x, residual, mod = aligned(x), aligned(residual), aligned(mod)
    B, S, Dx = x.shape
    h = torch.empty_like(x)
    out = torch.empty_like(x)
    mean = torch.empty((B, S), dtype=torch.float32, device=x.device)
    rstd = torch.empty((B, S), dtype=torch.float32, device=x.device)
    _call((x, residual, mod, h, out, mean, rstd), "adaln_residual_fwd", x.data_ptr(), residual.data_ptr(),
          mod.data_ptr(), h.data_ptr(), out.data_ptr(), mean.data_ptr(), rstd.data_ptr(), B, S, Dx, float(eps),
          _stream(x.device))
    return out, h, mean, rstd


def residual_bwd(g_out: torch.Tensor, g_h: torch.Tensor, x: torch.Tensor, h: torch.Tensor, mean: torch.Tensor,
                 rstd: torch.Tensor, mod: torch.Tensor):
    """Backward of the residual norm site (adaln_residual_bwd):
    (d_residual bf16, dx bf16, d_mod fp32 [B, 3 * 3072] = (d_shift | d_scale | d_gate))."""
    B, S = _rows(x)
    for t, n in ((g_out, "g_out"), (g_h, "g_h"), (h, "h")):
        _shape(t, x.shape, n)
    _shape(mean, (B, S), "mean")
    _shape(rstd, (B, S), "rstd")
    _shape(mod, (B, 3 * D), "mod")
    for t, n, dt in ((g_out, "g_out", torch.bfloat16), (g_h, "g_h", torch.bfloat16), (x, "x", torch.bfloat16),
                     (h, "h", torch.bfloat16), (mean, "mean", torch.float32), (rstd, "rstd", torch.float32),
                     (mod, "mod", torch.bfloat16)):
        _check(t, dt, n)
    g_out, g_h, x, h, mean, rstd, mod = (aligned(t) for t in (g_out, g_h, x, h, mean, rstd, mod))
    B, S, Dx = x.shape
    d_residual = torch.empty_like(x)
    dx = torch.empty_like(x)
    d_mod = torch.empty((B, 3 * Dx), dtype=torch.float32, device=x.device)
    ws = _ws(_lib.OP_RESIDUAL_BWD, B, S, Dx, x.device)
    _call((g_out, g_h, x, h, mean, rstd, mod, d_residual, dx, d_mod, ws), "adaln_residual_bwd", g_out.data_ptr(),
          g_h.data_ptr(), x.data_ptr(), h.data_ptr(), mean.data_ptr(), rstd.data_ptr(), mod.data_ptr(),
          d_residual.data_ptr(), dx.data_ptr(), d_mod.data_ptr(), ws.data_ptr(), ws.numel(), B, S, Dx,
          _stream(x.device))
    return d_residual, dx, d_mod


def _mod_views(views, dtype, name):
    """Three (or two) [B, D] views sharing one row stride, 16-byte aligned rows:
    (list of tensors, stride).  Otherwise copies them into one [B, n, D] buffer."""
    for v, n in zip(views, name):
        _check(v, dtype, n)
    el = views[0].element_size()
    ld = views[0].stride(0)
    ok = all(v.dim() == 2 and v.stride(1) == 1 and v.stride(0) == ld and v.data_ptr() % 16 == 0 for v in views)
    if ok and ld % 8 == 0 and (ld * el) % 16 == 0:
        return list(views), ld
    packed = torch.stack([v.contiguous() for v in views], dim=1)      # [B, n, D]
    return [packed[:, i] for i in range(len(views))], packed.stride(0)


def site_fwd(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, residual: torch.Tensor = None,
             gate: torch.Tensor = None, eps: float = EPS):
    """A block's norm site (adaln_site_fwd) with its modulation as [B, D] views,
    e.g. chunks of the 6-way projection's output.  residual None: the plain
    site, returns (out, mean, rstd); else the residual site h = bf16(residual +
    bf16(gate * x)), returns (out, h, mean, rstd)."""
    B, S = _rows(x)
    for v, n in ((shift, "shift"), (scale, "scale"), (gate, "gate")):
        if v is not None:
            _shape(v, (B, D), n)
    if residual is not None:
        _shape(residual, x.shape, "residual")
        if gate is None:
            raise ValueError("the residual form needs gate")
    _check(x, torch.bfloat16, "x")
    x = aligned(x)
    res = residual is not None
    views, ld = _mod_views([shift, scale] + ([gate] if res else []), torch.bfloat16, ("shift", "scale", "gate"))
    B, S, Dx = x.shape
    out = torch.empty_like(x)
    h = torch.empty_like(x) if res else None
    mean = torch.empty((B, S), dtype=torch.float32, device=x.device)
    rstd = torch.empty((B, S), dtype=torch.float32, device=x.device)
    if res:
        _check(residual, torch.bfloat16, "residual")
        residual = aligned(residual)
    _call((x, residual, *views, h, out, mean, rstd), "adaln_site_fwd", x.data_ptr(),
          residual.data_ptr() if res else None, views[0].data_ptr(), views[1].data_ptr(),
          views[2].data_ptr() if res else None, ld, h.data_ptr() if res else None, out.data_ptr(), mean.data_ptr(),
          rstd.data_ptr(), B, S, Dx, float(eps), _stream(x.device))
    return (out, h, mean, rstd) if res else (out, mean, rstd)


def site_bwd(g_out: torch.Tensor, x: torch.Tensor, mean: torch.Tensor, rstd: torch.Tensor, scale: torch.Tensor,
             g_h: torch.Tensor = None, h: torch.Tensor = None, gate: torch.Tensor = None, d_views=None):
    """Backward of a norm site (adaln_site_bwd).  g_h None: the plain site,
    returns (dx, d_shift, d_scale); else the residual site, returns
    (d_residual, dx, d_shift, d_scale, d_gate).  d_views: optional fp32 [B, D]
    output views (d_shift, d_scale[, d_gate]) with one row stride, e.g. chunks
    of a 6-way gradient; fresh tensors otherwise."""
    B, S = _rows(x)
    _shape(g_out, x.shape, "g_out")
    _shape(mean, (B, S), "mean")
    _shape(rstd, (B, S), "rstd")
    _shape(scale, (B, D), "scale")
    if g_h is not None:
        if h is None or gate is None:
            raise ValueError("the residual form needs h and gate")
        _shape(g_h, x.shape, "g_h")
        _shape(h, x.shape, "h")
        _shape(gate, (B, D), "gate")
    if d_views is not None:
        if len(d_views) != (3 if g_h is not None else 2):
            raise ValueError("d_views must hold one view per gradient (d_shift, d_scale[, d_gate])")
        for v in d_views:
            _shape(v, (B, D), "d_views")
    res = g_h is not None
    for t, n, dt in ((g_out, "g_out", torch.bfloat16), (x, "x", torch.bfloat16), (mean, "mean", torch.float32),
                     (rstd, "rstd", torch.float32)):
        _check(t, dt, n)
    g_out, x, mean, rstd = (aligned(t) for t in (g_out, x, mean, rstd))
    views, ld = _mod_views([scale] + ([gate] if res else []), torch.bfloat16, ("scale", "gate"))
    B, S, Dx = x.shape
    nseg = 3 if res else 2
    if d_views is None:
        dm = torch.empty((B, nseg, Dx), dtype=torch.float32, device=x.device)
        d_views = [dm[:, i] for i in range(nseg)]
    for v in d_views:
        _check(v, torch.float32, "d_views")
    dld = d_views[0].stride(0)
    if not all(v.stride(0) == dld and v.stride(1) == 1 and v.data_ptr() % 16 == 0 for v in d_views):
        raise ValueError("d_views must share one row stride and have 16-byte aligned rows")
    dx = torch.empty_like(x)
    d_res = None
    if res:
        _check(g_h, torch.bfloat16, "g_h")
        _check(h, torch.bfloat16, "h")
        g_h, h = aligned(g_h), aligned(h)
        d_res = torch.empty_like(x)
    ws = _ws(_lib.OP_RESIDUAL_BWD, B, S, Dx, x.device)
    _call((g_out, g_h, x, h, mean, rstd, *views, d_res, dx, *d_views, ws), "adaln_site_bwd", g_out.data_ptr(),
          g_h.data_ptr() if res else None, x.data_ptr(), h.data_ptr() if res else None, mean.data_ptr(),
          rstd.data_ptr(), views[0].data_ptr(), views[1].data_ptr() if res else None, ld,
          d_res.data_ptr() if res else None, dx.data_ptr(), d_views[0].data_ptr(), d_views[1].data_ptr(),
          d_views[2].data_ptr() if res else None, dld, ws.data_ptr(), ws.numel(), B, S, Dx, _stream(x.device))
    if res:
        return d_res, dx, d_views[0], d_views[1], d_views[2]
    return dx, d_views[0], d_views[1]


def proj_out_fwd(out: torch.Tensor, W: torch.Tensor, bias: torch.Tensor) -> torch.Tensor:
    """proj_out (adaln_proj_out_fwd): latent [..., 64] bf16 = bf16(out W^T + b) per
    token; out [..., 3072], W [64, 3072], bias [64], all bf16."""
    if out.dim() < 1 or out.shape[-1] != D:
        raise ValueError(f"out must have shape (..., {D}), got {tuple(out.shape)}")
    _shape(W, (64, D), "W")
    _shape(bias, (64,), "bias")
    for t, n in ((out, "out"), (W, "W"), (bias, "bias")):
        _check(t, torch.bfloat16, n)
    out, W, bias = aligned(out), aligned(W), aligned(bias)
    T = out.numel() // out.shape[-1]
    latent = torch.empty(out.shape[:-1] + (W.shape[0],), dtype=torch.bfloat16, device=out.device)
    B, S = (out.shape[0], out.shape[1]) if out.dim() == 3 else (1, T)   # the workspace depends on T = B * S
    ws = _ws(_lib.OP_PROJ_OUT_FWD, B, S, out.shape[-1], out.device)
    _call((out, W, bias, latent, ws), "adaln_proj_out_fwd", out.data_ptr(), W.data_ptr(), bias.data_ptr(),
          latent.data_ptr(), ws.data_ptr(), ws.numel(), T, out.shape[-1], W.shape[0], _stream(out.device))
    return latent


def fwd_proj_out(x: torch.Tensor, temb: torch.Tensor, W: torch.Tensor, bias: torch.Tensor, Wp: torch.Tensor,
                 bp: torch.Tensor, eps: float = EPS):
    """Serving forward of the final layer (adaln_fwd_proj_out): the final
    modulation then proj_out without the modulated output in memory.  Returns
    (latent [B, S, 64], emb, mean, rstd), the same bits as fwd followed by
    proj_out_fwd on its out.  All tensors bf16."""
    B, S = _rows(x)
    _shape(temb, (B, D), "temb")
    _proj_width(W, (N,))
    _shape(bias, (N,), "bias")
    _shape(Wp, (64, D), "Wp")
    _shape(bp, (64,), "bp")
    for t, n in ((x, "x"), (temb, "temb"), (W, "W"), (bias, "bias"), (Wp, "Wp"), (bp, "bp")):
        _check(t, torch.bfloat16, n)
    x, temb, W, bias, Wp, bp = (aligned(t) for t in (x, temb, W, bias, Wp, bp))
    B, S, Dx = x.shape
    emb = torch.empty((B, N), dtype=torch.bfloat16, device=x.device)
    latent = torch.empty((B, S, Wp.shape[0]), dtype=torch.bfloat16, device=x.device)
    mean = torch.empty((B, S), dtype=torch.float32, device=x.device)
    rstd = torch.empty((B, S), dtype=torch.float32, device=x.device)
    ws = _ws(_lib.OP_FWD_PROJ_OUT, B, S, Dx, x.device)
    _call((temb, W, bias, x, Wp, bp, emb, latent, mean, rstd, ws), "adaln_fwd_proj_out", temb.data_ptr(),
          W.data_ptr(), bias.data_ptr(), x.data_ptr(), Wp.data_ptr(), bp.data_ptr(), emb.data_ptr(),
          latent.data_ptr(), mean.data_ptr(), rstd.data_ptr(), ws.data_ptr(), ws.numel(), B, S, Dx, Wp.shape[0],
          float(eps), _stream(x.device))
    return latent, emb, mean, rstd


def proj_out_bwd(d_lat: torch.Tensor, out: torch.Tensor, W: torch.Tensor):
    """Backward of proj_out (adaln_proj_out_bwd): (d_out bf16 like out, dW bf16
    [64, 3072], db bf16 [64])."""
    if out.dim() < 1 or out.shape[-1] != D:
        raise ValueError(f"out must have shape (..., {D}), got {tuple(out.shape)}")
    _shape(W, (64, D), "W")
    _shape(d_lat, tuple(out.shape[:-1]) + (64,), "d_lat")
    for t, n in ((d_lat, "d_lat"), (out, "out"), (W, "W")):
        _check(t, torch.bfloat16, n)
    d_lat, out, W = aligned(d_lat), aligned(out), aligned(W)
    T = out.numel() // out.shape[-1]
    d_out = torch.empty_like(out)
    dW = torch.empty_like(W)
    db = torch.empty((W.shape[0],), dtype=torch.bfloat16, device=W.device)
    B, S = (out.shape[0], out.shape[1]) if out.dim() == 3 else (1, T)   # the workspace depends on T = B * S
    ws = _ws(_lib.OP_PROJ_OUT_BWD, B, S, out.shape[-1], out.device)
    _call((d_lat, out, W, d_out, dW, db, ws), "adaln_proj_out_bwd", d_lat.data_ptr(), out.data_ptr(), W.data_ptr(),
          d_out.data_ptr(), dW.data_ptr(), db.data_ptr(), ws.data_ptr(), ws.numel(), T, out.shape[-1], W.shape[0],
          _stream(out.device))
    return d_out, dW, db


def selftest() -> int:
    return int(_lib.load().adaln_selftest())


class AdaLNFinal(torch.autograd.Function):
    """out = LayerNorm(x) * (1 + scale) + shift with (scale, shift) = (SiLU(temb) W^T + b).chunk(2).

    Inputs: x [B, S, 3072], temb [B, 3072], W [6144, 3072], b [6144], all bf16
    (the autocast rounding points) or all fp32 (fp32 storage).  Saves x, temb,
    W, emb, mean and rstd (8 bytes per row of LayerNorm state, not the
    normalized activations)."""

    @staticmethod
    def forward(ctx, x, temb, W, b, eps=EPS):
        out, emb, mean, rstd = fwd(x, temb, W, b, eps)
        ctx.save_for_backward(x, temb, W, emb, mean, rstd)
        return out

    @staticmethod
    def backward(ctx, g):
        x, temb, W, emb, mean, rstd = ctx.saved_tensors
        if g.dtype != x.dtype:
            raise TypeError(f"the upstream gradient must be {x.dtype} (the output's dtype), got {g.dtype}")
        dx, d_emb, dW, db, dtemb = bwd(g, x, mean, rstd, emb, temb, W)
        return dx, dtemb, dW, db, None


def adaln_final(x, temb, W, b, eps=EPS):
    return AdaLNFinal.apply(x, temb, W, b, eps)


class ProjOut(torch.autograd.Function):
    """latent = out Wp^T + bp per token (proj_out, 3072 -> 64), bf16; saves out and Wp."""

    @staticmethod
    def forward(ctx, out, Wp, bp):
        ctx.save_for_backward(out, Wp)
        return proj_out_fwd(out, Wp, bp)

    @staticmethod
    def backward(ctx, g):
        out, Wp = ctx.saved_tensors
        if g.dtype != torch.bfloat16:
            raise TypeError(f"the upstream gradient must be torch.bfloat16 (latent's dtype), got {g.dtype}")
        d_out, dW, db = proj_out_bwd(g, out, Wp)
        return d_out, dW, db


def proj_out(out, Wp, bp):
    return ProjOut.apply(out, Wp, bp)
