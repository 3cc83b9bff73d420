"""The largest shapes the C ABI accepts (include/adaln.h: B <= 65535, S <= 32 x
65535), run through the one-call entry points and the residual site; proj_out
at 2^22 tokens.

The oracle cannot evaluate these sizes whole, so the checks are ones that hold
at any size: d_shift columns (the token tree at its deepest, four levels above
the tiles) against the CPU tree model on the same column of g, and per-row /
per-sample outputs against small runs holding the same rows or samples (rows
depend only on their own data and on emb; samples only on their own data).
Inputs are drawn on the GPU from a seeded generator; only slices come back.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import token_tree
from synthetic_inputs import make_inputs
from tests.gpu_helpers import same_bytes, to_dev

pytestmark = pytest.mark.gpu

D = 3072


def _params(seed: int):
    inp = make_inputs(1, 1, seed=seed)
    return to_dev(inp["temb"]), to_dev(inp["W"]), to_dev(inp["bias"])


def _randn(shape, gen):
    return torch.randn(shape, device="cuda", generator=gen).to(torch.bfloat16)


def test_maximum_sequence_length(gpu_lib):
    from invariant_silu_amd import ops
    S = 32 * 65535
    print(f"[limits] B=1 S={S}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(2026)
    x = _randn((1, S, D), gen)
    g = _randn((1, S, D), gen)
    temb, W, bias = _params(41)
    out, emb, mean, rstd = ops.fwd(x, temb, W, bias)
    dx, d_emb, dW, db, dtemb = ops.bwd(g, x, mean, rstd, emb, temb, W)
    torch.cuda.synchronize()
    cols = [0, 1, 1000, 3071]
    gcols = g[0][:, cols].float().cpu().numpy()                     # [S, 4], exact widening
    want = token_tree.tree_sum(gcols[None])[0]
    got = d_emb[0, [D + c for c in cols]].cpu().numpy()
    assert got.tobytes() == want.tobytes()
    # rows of the long run against a 40-token run holding the same rows
    rows = torch.tensor([0, 1, 31, 32, 33, 4095, 4096, 1048575, 1048576, 2000001] + list(range(S - 30, S)),
                        device="cuda")
    xs, gs = x[:, rows].contiguous(), g[:, rows].contiguous()
    o2, e2, m2, r2 = ops.fwd(xs, temb, W, bias)
    dx2, _, _, _, _ = ops.bwd(gs, xs, m2, r2, e2, temb, W)
    assert same_bytes(e2, emb)
    assert same_bytes(o2, out[:, rows]) and same_bytes(dx2, dx[:, rows])
    assert same_bytes(m2, mean[:, rows]) and same_bytes(r2, rstd[:, rows])
    del x, g, out, dx


def test_maximum_batch(gpu_lib):
    from invariant_silu_amd import ops
    B = 65535
    print(f"[limits] B={B} S=1", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(127)
    x = _randn((B, 1, D), gen)
    g = _randn((B, 1, D), gen)
    temb = _randn((B, D), gen)
    _, W, bias = _params(43)
    out, emb, mean, rstd = ops.fwd(x, temb, W, bias)
    dx, d_emb, dW, db, dtemb = ops.bwd(g, x, mean, rstd, emb, temb, W)
    full = dict(out=out, emb=emb, mean=mean, rstd=rstd, dx=dx, d_emb=d_emb, dtemb=dtemb)
    for b in (0, 1, 15, 16, 4095, 32767, 65519, 65534):
        o1, e1, m1, r1 = ops.fwd(x[b:b + 1], temb[b:b + 1], W, bias)
        dx1, de1, _, _, dt1 = ops.bwd(g[b:b + 1], x[b:b + 1], m1, r1, e1, temb[b:b + 1], W)
        one = dict(out=o1, emb=e1, mean=m1, rstd=r1, dx=dx1, d_emb=de1, dtemb=dt1)
        for k, v in one.items():
            assert same_bytes(full[k][b:b + 1], v), f"sample {b} {k}"
    assert torch.isfinite(dW.float()).all() and torch.isfinite(db.float()).all()


def _site_inputs(shape, gen):
    return {k: _randn(shape, gen) for k in ("x", "residual", "g_out", "g_h")}


def test_residual_site_maximum_sequence_length(gpu_lib):
    """The residual site at S = 32 x 65535 (four tree levels): d_shift columns
    against the CPU tree model, sampled rows against a short run holding them."""
    from invariant_silu_amd import ops
    S = 32 * 65535
    print(f"[limits] residual site B=1 S={S}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(31)
    d = _site_inputs((1, S, D), gen)
    mod = (torch.randn((1, 3 * D), device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    out, h, mean, rstd = ops.residual_fwd(d["x"], d["residual"], mod)
    d_res, dx, d_mod = ops.residual_bwd(d["g_out"], d["g_h"], d["x"], h, mean, rstd, mod)
    torch.cuda.synchronize()
    cols = [0, 1, 1000, 3071]
    want = token_tree.tree_sum(d["g_out"][0][:, cols].float().cpu().numpy()[None])[0]
    assert d_mod[0, cols].cpu().numpy().tobytes() == want.tobytes()
    rows = torch.tensor([0, 31, 32, 4096, 1048576, 2000001] + list(range(S - 20, S)), device="cuda")
    sub = {k: v[:, rows].contiguous() for k, v in d.items()}
    o2, h2, m2, r2 = ops.residual_fwd(sub["x"], sub["residual"], mod)
    dr2, dx2, _ = ops.residual_bwd(sub["g_out"], sub["g_h"], sub["x"], h2, m2, r2, mod)
    for a, b in ((o2, out), (h2, h), (m2, mean), (r2, rstd), (dr2, d_res), (dx2, dx)):
        assert same_bytes(a, b[:, rows])
    del d, out, h, d_res, dx


def test_residual_site_maximum_batch(gpu_lib):
    """The residual site at B = 65535, S = 1: sampled samples against runs of one."""
    from invariant_silu_amd import ops
    B = 65535
    print(f"[limits] residual site B={B} S=1", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(32)
    d = _site_inputs((B, 1, D), gen)
    mod = (torch.randn((B, 3 * D), device="cuda", generator=gen) * 0.5).to(torch.bfloat16)
    out, h, mean, rstd = ops.residual_fwd(d["x"], d["residual"], mod)
    d_res, dx, d_mod = ops.residual_bwd(d["g_out"], d["g_h"], d["x"], h, mean, rstd, mod)
    full = dict(out=out, h=h, mean=mean, rstd=rstd, d_res=d_res, dx=dx, d_mod=d_mod)
    for b in (0, 1, 4095, 32767, 65519, 65534):
        s = {k: v[b:b + 1] for k, v in d.items()}
        o1, h1, m1, r1 = ops.residual_fwd(s["x"], s["residual"], mod[b:b + 1])
        dr1, dx1, dm1 = ops.residual_bwd(s["g_out"], s["g_h"], s["x"], h1, m1, r1, mod[b:b + 1])
        one = dict(out=o1, h=h1, mean=m1, rstd=r1, d_res=dr1, dx=dx1, d_mod=dm1)
        for k, v in one.items():
            assert same_bytes(full[k][b:b + 1], v), f"sample {b} {k}"


def test_proj_out_large_token_count(gpu_lib):
    """proj_out at T = 2^22 tokens: sampled tokens' latent and d_out against the
    oracle (a token's outputs depend only on its own row); dWp, dbp finite."""
    from invariant_silu_amd import ops
    from oracle import proj_out as po
    from tests.compare import bf16_gate
    from tests.gpu_helpers import bf16_bits
    T = 1 << 22
    print(f"[limits] proj_out T={T}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(33)
    out = _randn((T, D), gen)
    d_lat = _randn((T, 64), gen)
    W = (torch.randn((64, D), device="cuda", generator=gen) * 0.02).to(torch.bfloat16)
    bias = (torch.randn((64,), device="cuda", generator=gen) * 0.01).to(torch.bfloat16)
    latent = ops.proj_out_fwd(out, W, bias)
    d_out, dW, db = ops.proj_out_bwd(d_lat, out, W)
    torch.cuda.synchronize()
    rows = torch.tensor([0, 1, 511, 512, 1 << 20, T - 2, T - 1], device="cuda")
    sub = {"out": bf16_bits(out[rows]), "W": bf16_bits(W), "bias": bf16_bits(bias), "d_lat": bf16_bits(d_lat[rows])}
    f, f6 = (po.proj_out_forward(sub, m) for m in ("fp32", "fp64"))
    b, b6 = (po.proj_out_backward(sub, m, outputs=("d_out",)) for m in ("fp32", "fp64"))
    r = bf16_gate(bf16_bits(latent[rows]), f["latent_bits"], f6["latent_bits"])
    assert r["n_fail"] == 0, r
    r = bf16_gate(bf16_bits(d_out[rows]), b["d_out_bits"], b6["d_out_bits"])
    assert r["n_fail"] == 0, r
    assert torch.isfinite(dW.float()).all() and torch.isfinite(db.float()).all()
    del out, d_out
