"""FP32 storage on the GPU: parity with the oracle's fp32 storage mode and
bytewise batch invariance (RL-Kernel pull request 538 measures and gates the
operator in FP32 beside BF16: "Prior art & reuse decision", "Results").

fp32 outputs are gated as |gpu - o| <= 1e-5 |o| + 2^-24 A (tests/compare.py),
with A the sum of |terms| for the reduced outputs (the oracle returns it) and,
for the elementwise ones, 16 times the magnitude of the expression's operands
(a few fp32 ulps of them, which covers one-ulp differences of the statistics
or of emb they are computed from).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import adaln
from synthetic_inputs import make_inputs
from tests.compare import f32_gate

pytestmark = pytest.mark.gpu

ROW_KEYS = ("emb", "out", "mean", "rstd", "dx", "d_emb", "dtemb")


def _dev(inp: dict) -> dict:
    return {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda() for k in ("x", "temb", "W", "bias", "g")}


def _run(d: dict) -> dict:
    from invariant_silu_amd import ops
    out, emb, mean, rstd = ops.fwd(d["x"], d["temb"], d["W"], d["bias"])
    dx, d_emb, dW, db, dtemb = ops.bwd(d["g"], d["x"], mean, rstd, emb, d["temb"], d["W"])
    return dict(emb=emb, out=out, mean=mean, rstd=rstd, dx=dx, d_emb=d_emb, dW=dW, db=db, dtemb=dtemb)


def _host(r: dict) -> dict:
    torch.cuda.synchronize()
    return {k: v.detach().cpu().numpy() for k, v in r.items()}


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return a.shape == b.shape and bool(torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32)))


@pytest.mark.parametrize("B,S", [(1, 31), (2, 64), (5, 17), (6, 40), (1, 6032), (2, 6889)])
def test_fp32_parity(gpu_lib, B, S):
    """Small shapes on both projection paths, and the pages' long-sequence
    shapes (S = 6032, 6889: several levels of the token tree)."""
    print(f"[fp32] parity B={B} S={S}", flush=True)
    inp = make_inputs(B, S, seed=B * 100 + S, outlier_frac=0.05, io="fp32")
    gpu = _host(_run(_dev(inp)))
    f = adaln.forward(inp, want_abs=True)
    b = adaln.backward(inp, f, want_abs=True)
    n, m = f["n"].astype(np.float64), f["m"].astype(np.float64)
    shift = f["emb"][:, 3072:].astype(np.float64)
    A_out = 16 * (np.abs(n * m[:, None, :]) + np.abs(shift[:, None, :]))
    g = inp["g"].astype(np.float64)
    gy = g * m[:, None, :]
    rs = f["rstd"][..., None].astype(np.float64)
    al, be = b["alpha"][..., None].astype(np.float64), b["beta"][..., None].astype(np.float64)
    A_dx = 16 * rs * (np.abs(gy) + np.abs(al) + np.abs(n * be))
    ds = np.abs(adaln.dsilu(inp["temb"], adaln.Arith("fp32")).astype(np.float64))
    checks = {
        "emb": (f["emb"], f["A_emb"]),
        "out": (f["out"], A_out),
        "rstd": (f["rstd"], np.zeros_like(f["rstd"], dtype=np.float64)),
        "dx": (b["dx"], A_dx),
        "d_emb": (b["d_emb"], b["A_d_emb"]),
        "dtemb": (b["dtemb"], 16 * b["A_da"] * ds),
        "dW": (b["dW"], b["A_dW"]),
        "db": (b["db"], b["A_db"]),
    }
    for k, (o, A) in checks.items():
        r = f32_gate(gpu[k], o, A)
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k


@pytest.mark.parametrize("B,S", [(5, 33), (20, 3), (70, 2)])
def test_fp32_singleton_vs_batch(gpu_lib, B, S):
    """Per-sample outputs are the same bytes alone (B = 1: vector da) and in
    the batch (B > 4: matrix-core da)."""
    print(f"[fp32] invariance B={B} S={S}", flush=True)
    d = _dev(make_inputs(B, S, seed=7, io="fp32"))
    full = _run(d)
    for bi in range(B):
        one = _run({k: (v[bi:bi + 1] if k in ("x", "temb", "g") else v) for k, v in d.items()})
        for k in ROW_KEYS:
            assert _same(full[k][bi:bi + 1], one[k]), f"sample {bi} {k}"
    # B = 4 (vector da) against the same rows of the batch
    four = _run({k: (v[:4] if k in ("x", "temb", "g") else v) for k, v in d.items()})
    for k in ROW_KEYS:
        assert _same(full[k][:4], four[k]), k


def test_fp32_param_grads_zero_padding(gpu_lib):
    """dW and db are unchanged by trailing samples whose upstream gradient is zero."""
    print("[fp32] ordered zero padding", flush=True)
    d = _dev(make_inputs(6, 40, seed=9, io="fp32"))
    base = _run({k: (v[:3] if k in ("x", "temb", "g") else v) for k, v in d.items()})
    padded = dict(d)
    padded["g"] = d["g"].clone()
    padded["g"][3:] = 0
    r = _run(padded)
    assert _same(r["dW"], base["dW"]) and _same(r["db"], base["db"])


def test_fp32_autograd(gpu_lib):
    """AdaLNFinal with fp32 tensors gives the one-call results."""
    print("[fp32] autograd", flush=True)
    from invariant_silu_amd import ops
    d = _dev(make_inputs(2, 24, seed=11, io="fp32"))
    x, temb, W, b = (d[k].clone().requires_grad_(True) for k in ("x", "temb", "W", "bias"))
    out = ops.adaln_final(x, temb, W, b)
    out.backward(d["g"])
    ref = _run(d)
    assert _same(out.detach(), ref["out"])
    assert _same(x.grad, ref["dx"]) and _same(temb.grad, ref["dtemb"])
    assert _same(W.grad, ref["dW"]) and _same(b.grad, ref["db"])
