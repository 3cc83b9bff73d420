"""A block's norm sites with their modulation as views (adaln_site_fwd /
adaln_site_bwd), fed straight from a 6-way modulation tensor [B, 6D] =
(shift1 | scale1 | gate1 | shift2 | scale2 | gate2) and writing gradients into
a 6-way gradient tensor.

The plain site must give the bytes of the final modulation's kernels with emb =
(scale | shift) (adaln_norm_mod_fwd / _bwd, parity-tested against the oracle
in test_gpu_parity.py) and, directly, the oracle's (the plain site is the
final modulation's norm and modulation, oracle/adaln.py, with W = 0 so that
emb = bias = (scale | shift)); the residual site with views must give the
bytes of adaln_residual_fwd / _bwd on the same chunks copied into one
contiguous (shift | scale | gate) (parity-tested in test_gpu_residual.py).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import adaln
from synthetic_inputs import make_residual_inputs
from tests.compare import bf16_gate, f32_gate
from tests.gpu_helpers import bf16_bits, same_bytes, to_dev

pytestmark = pytest.mark.gpu

D = 3072


def _mod6(B, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn((B, 6 * D), device="cuda", generator=g) * 0.5).to(torch.bfloat16)


def _chunk(t, q):
    return t[:, q * D:(q + 1) * D]


@pytest.mark.parametrize("B,S", [(1, 31), (3, 70)])
def test_plain_site_equals_final_modulation(gpu_lib, B, S):
    """Site 1 (shift1, scale1 from the 6-way tensor) against adaln_norm_mod_* with
    emb = (scale1 | shift1): the same bytes for out, mean, rstd, dx, d_shift and
    d_scale (written into the 6-way gradient at chunks 0 and 1)."""
    print(f"[site] plain B={B} S={S}", flush=True)
    from invariant_silu_amd import ops
    inp = make_residual_inputs(B, S, seed=130 + S)
    x, g = to_dev(inp["x"]), to_dev(inp["g_out"])
    mod6 = _mod6(B, 131)
    shift1, scale1 = _chunk(mod6, 0), _chunk(mod6, 1)
    out, mean, rstd = ops.site_fwd(x, shift1, scale1)
    emb = torch.cat([scale1, shift1], dim=1).contiguous()
    out2, mean2, rstd2 = ops.norm_mod_fwd(x, emb)
    assert same_bytes(out, out2) and same_bytes(mean, mean2) and same_bytes(rstd, rstd2)
    dmod6 = torch.full((B, 6 * D), float("nan"), dtype=torch.float32, device="cuda")
    dx, d_shift, d_scale = ops.site_bwd(g, x, mean, rstd, scale1, d_views=[_chunk(dmod6, 0), _chunk(dmod6, 1)])
    dx2, d_emb2 = ops.norm_mod_bwd(g, x, mean2, rstd2, emb)
    assert same_bytes(dx, dx2)
    assert same_bytes(_chunk(dmod6, 1).contiguous(), d_emb2[:, :D].contiguous())    # d_scale
    assert same_bytes(_chunk(dmod6, 0).contiguous(), d_emb2[:, D:].contiguous())    # d_shift
    assert torch.isnan(dmod6[:, 2 * D:]).all()                                       # other chunks untouched


def test_plain_site_oracle(gpu_lib):
    """The plain site against the oracle (final modulation with W = 0, emb = bias
    = (scale | shift))."""
    print("[site] plain oracle", flush=True)
    from invariant_silu_amd import ops
    B, S = 2, 45
    inp = make_residual_inputs(B, S, seed=140)
    mod6 = _mod6(B, 141)
    shift1, scale1 = _chunk(mod6, 0), _chunk(mod6, 1)
    x, g = to_dev(inp["x"]), to_dev(inp["g_out"])
    out, mean, rstd = ops.site_fwd(x, shift1, scale1)
    dx, d_shift, d_scale = ops.site_bwd(g, x, mean, rstd, scale1)
    torch.cuda.synchronize()
    emb_bits = bf16_bits(torch.cat([scale1, shift1], dim=1).contiguous())
    oinp = {"x": inp["x"], "g": inp["g_out"], "temb": np.zeros((B, D), np.uint16),
            "W": np.zeros((2 * D, D), np.uint16), "bias": emb_bits[0]}
    for b in range(B):   # the oracle's bias is one row: one sample at a time
        ob = {k: (v[b:b + 1] if k in ("x", "g", "temb") else v) for k, v in oinp.items()}
        ob["bias"] = emb_bits[b]
        f = adaln.forward(ob)
        bw = adaln.backward(ob, f, want_abs=True)
        f6 = adaln.forward(ob, "fp64")
        b6 = adaln.backward(ob, f6, "fp64")
        assert bf16_gate(bf16_bits(out[b:b + 1]), f["out_bits"], f6["out_bits"])["n_fail"] == 0
        assert bf16_gate(bf16_bits(dx[b:b + 1]), bw["dx_bits"], b6["dx_bits"])["n_fail"] == 0
        A = bw["A_d_emb"]
        r1 = f32_gate(d_scale[b:b + 1].cpu().numpy(), bw["d_emb"][:, :D], A[:, :D])
        r2 = f32_gate(d_shift[b:b + 1].cpu().numpy(), bw["d_emb"][:, D:], A[:, D:])
        print(f"  sample {b}: d_scale {r1['n_fail']} d_shift {r2['n_fail']}")
        assert r1["n_fail"] == 0 and r2["n_fail"] == 0


@pytest.mark.parametrize("B,S", [(1, 33), (2, 64)])
def test_residual_site_views_equal_contiguous(gpu_lib, B, S):
    """Site 2 of a block: gate1 with shift2, scale2 as views of the 6-way tensor,
    gradients into chunks 2, 3, 4 of a 6-way gradient, against
    adaln_residual_* on cat(shift2, scale2, gate1)."""
    print(f"[site] residual views B={B} S={S}", flush=True)
    from invariant_silu_amd import ops
    inp = make_residual_inputs(B, S, seed=150 + S)
    d = {k: to_dev(inp[k]) for k in ("x", "residual", "g_out", "g_h")}
    mod6 = _mod6(B, 151)
    shift2, scale2, gate1 = _chunk(mod6, 3), _chunk(mod6, 4), _chunk(mod6, 2)
    out, h, mean, rstd = ops.site_fwd(d["x"], shift2, scale2, residual=d["residual"], gate=gate1)
    mod = torch.cat([shift2, scale2, gate1], dim=1).contiguous()
    out2, h2, mean2, rstd2 = ops.residual_fwd(d["x"], d["residual"], mod)
    for a, b in ((out, out2), (h, h2), (mean, mean2), (rstd, rstd2)):
        assert same_bytes(a, b)
    dmod6 = torch.full((B, 6 * D), float("nan"), dtype=torch.float32, device="cuda")
    views = [_chunk(dmod6, 3), _chunk(dmod6, 4), _chunk(dmod6, 2)]     # d_shift2, d_scale2, d_gate1
    d_res, dx, _, _, _ = ops.site_bwd(d["g_out"], d["x"], mean, rstd, scale2, g_h=d["g_h"], h=h, gate=gate1,
                                      d_views=views)
    d_res2, dx2, d_mod2 = ops.residual_bwd(d["g_out"], d["g_h"], d["x"], h2, mean2, rstd2, mod)
    assert same_bytes(d_res, d_res2) and same_bytes(dx, dx2)
    for v, q in ((views[0], 0), (views[1], 1), (views[2], 2)):
        assert same_bytes(v.contiguous(), d_mod2[:, q * D:(q + 1) * D].contiguous()), q
    assert torch.isnan(dmod6[:, :2 * D]).all() and torch.isnan(dmod6[:, 5 * D:]).all()


def test_site_batch_invariance(gpu_lib):
    """Per-sample outputs of both site forms are the same bytes alone and in a
    batch of 5 with views of one 6-way tensor."""
    print("[site] invariance", flush=True)
    from invariant_silu_amd import ops
    B, S = 5, 40
    inp = make_residual_inputs(B, S, seed=160)
    d = {k: to_dev(inp[k]) for k in ("x", "residual", "g_out", "g_h")}
    mod6 = _mod6(B, 161)

    def run(sl):
        m = mod6[sl]
        x, r, g, gh = (d[k][sl] for k in ("x", "residual", "g_out", "g_h"))
        o1, mu1, rs1 = ops.site_fwd(x, _chunk(m, 0), _chunk(m, 1))
        dx1, ds1, dc1 = ops.site_bwd(g, x, mu1, rs1, _chunk(m, 1))
        o2, h2, mu2, rs2 = ops.site_fwd(x, _chunk(m, 3), _chunk(m, 4), residual=r, gate=_chunk(m, 2))
        dr2, dx2, ds2, dc2, dg2 = ops.site_bwd(g, x, mu2, rs2, _chunk(m, 4), g_h=gh, h=h2, gate=_chunk(m, 2))
        return [o1, dx1, ds1, dc1, o2, h2, dr2, dx2, ds2, dc2, dg2]

    full = run(slice(0, B))
    for b in range(B):
        one = run(slice(b, b + 1))
        for i, (a, o) in enumerate(zip(full, one)):
            assert same_bytes(a[b:b + 1].contiguous(), o.contiguous()), (b, i)
