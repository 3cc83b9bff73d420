"""The largest shapes the C ABI accepts (include/adaln.h: B <= 65535, S <= 32 x
65535), run through the one-call entry points.

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
