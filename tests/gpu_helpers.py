"""Helpers for the GPU tests: move seeded bf16 inputs to the device, run the
HIP path through the C ABI (via invariant_silu_amd.ops), bring outputs back."""

from __future__ import annotations

import numpy as np
import torch

from invariant_silu_amd import ops

KEYS_BF16 = ("emb", "out", "dx", "dtemb", "dW", "db")
KEYS_F32 = ("mean", "rstd", "d_emb")
ROW_KEYS = ("emb", "out", "mean", "rstd", "dx", "d_emb", "dtemb")   # per-sample outputs


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_vals(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def dev_inputs(inp: dict) -> dict:
    return {k: to_dev(inp[k]) for k in ("x", "temb", "W", "bias", "g")}


def run_path_dev(d: dict, eps: float = 1e-6) -> dict:
    """Forward + backward on device tensors; returns device tensors."""
    emb = ops.proj_fwd(d["temb"], d["W"], d["bias"])
    out, mean, rstd = ops.norm_mod_fwd(d["x"], emb, eps)
    dx, d_emb = ops.norm_mod_bwd(d["g"], d["x"], mean, rstd, emb)
    dW, db, dtemb = ops.proj_bwd(d_emb, d["temb"], d["W"])
    return dict(emb=emb, out=out, mean=mean, rstd=rstd, dx=dx, d_emb=d_emb, dW=dW, db=db, dtemb=dtemb)


def run_onecall_dev(d: dict, eps: float = 1e-6) -> dict:
    """The same step through the one-call entry points adaln_fwd / adaln_bwd."""
    out, emb, mean, rstd = ops.fwd(d["x"], d["temb"], d["W"], d["bias"], eps)
    dx, d_emb, dW, db, dtemb = ops.bwd(d["g"], d["x"], mean, rstd, emb, d["temb"], d["W"])
    return dict(emb=emb, out=out, mean=mean, rstd=rstd, dx=dx, d_emb=d_emb, dW=dW, db=db, dtemb=dtemb)


def to_host(r: dict) -> dict:
    torch.cuda.synchronize()
    h = {}
    for k, v in r.items():
        h[k] = bf16_bits(v) if v.dtype == torch.bfloat16 else f32_vals(v)
    return h


def run_path(inp: dict, eps: float = 1e-6) -> dict:
    return to_host(run_path_dev(dev_inputs(inp), eps))


def same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.shape != b.shape or a.dtype != b.dtype:
        return False
    iv = torch.int16 if a.element_size() == 2 else torch.int32
    return bool(torch.equal(a.contiguous().view(iv), b.contiguous().view(iv)))
