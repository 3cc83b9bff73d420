"""proj_out (3072 -> 64 per token) on the GPU through adaln_proj_out_fwd /
adaln_proj_out_bwd: parity with oracle/proj_out.py, per-token invariance and
zero-gradient padding of dWp, dbp.

Gate (tests/compare.py, bf16_gate): every bf16 output within 1 ulp of the
fp32 oracle, else within 1 ulp of its fp64 twin -- the same bar as every other
bf16 output.  The kernels multiply exactly and accumulate in fp64 on the
matrix cores, so they land on the correctly rounded sums; the cases at T = 600
and T = 4096 are where the earlier fp32-accumulating bf16 kernels left
cancelling sums several ulps off.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import proj_out as po
from synthetic_inputs import make_proj_out_inputs
from tests.compare import bf16_gate
from tests.gpu_helpers import bf16_bits, same_bytes, to_dev

pytestmark = pytest.mark.gpu

K, O = 3072, 64


KEYS = ("out", "W", "bias", "d_lat")


def _inputs(T, seed):
    inp = make_proj_out_inputs(T, seed)
    return {k: inp[k] for k in KEYS}


def _run(d):
    from invariant_silu_amd import ops
    latent = ops.proj_out_fwd(d["out"], d["W"], d["bias"])
    d_out, dW, db = ops.proj_out_bwd(d["d_lat"], d["out"], d["W"])
    return dict(latent=latent, d_out=d_out, dW=dW, db=db)


@pytest.mark.parametrize("T", [1, 37, 511, 512, 513, 600])
def test_proj_out_parity(gpu_lib, T):
    print(f"[proj_out] parity T={T}", flush=True)
    inp = _inputs(T, seed=100 + T)
    gpu = _run({k: to_dev(v) for k, v in inp.items()})
    torch.cuda.synchronize()
    f, f6 = (po.proj_out_forward(inp, m) for m in ("fp32", "fp64"))
    b, b6 = (po.proj_out_backward(inp, m) for m in ("fp32", "fp64"))
    for k, o, t in (("latent", f, f6), ("d_out", b, b6), ("dW", b, b6), ("db", b, b6)):
        r = bf16_gate(bf16_bits(gpu[k]), o[k + "_bits"], t[k + "_bits"])
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k


def test_proj_out_large_sampled(gpu_lib):
    """T = 4096 (one 1024 x 1024 image stream): latent and d_out of sampled tokens
    (each token on its own in the oracle), dWp and dbp in full."""
    T = 4096
    print(f"[proj_out] T={T} sampled", flush=True)
    inp = _inputs(T, seed=111)
    gpu = _run({k: to_dev(v) for k, v in inp.items()})
    torch.cuda.synchronize()
    rows = np.array([0, 1, 15, 16, 63, 64, 511, 512, 2047, 4031, 4094, 4095])
    sub = dict(inp, out=inp["out"][rows], d_lat=inp["d_lat"][rows])
    f, f6 = (po.proj_out_forward(sub, m) for m in ("fp32", "fp64"))
    bs, bs6 = (po.proj_out_backward(sub, m, outputs=("d_out",)) for m in ("fp32", "fp64"))
    for k, got, o, t in (("latent", gpu["latent"][rows], f, f6), ("d_out", gpu["d_out"][rows], bs, bs6)):
        r = bf16_gate(bf16_bits(got), o[k + "_bits"], t[k + "_bits"])
        print(f"  {k} (sampled): {r}")
        assert r["n_fail"] == 0, k
    b, b6 = (po.proj_out_backward(inp, m, outputs=("dW", "db")) for m in ("fp32", "fp64"))
    for k in ("dW", "db"):
        r = bf16_gate(bf16_bits(gpu[k]), b[k + "_bits"], b6[k + "_bits"])
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k


def test_proj_out_token_invariance(gpu_lib):
    """latent and d_out of a token are the same bytes alone, in a ragged run and
    at any offset of a long run."""
    print("[proj_out] token invariance", flush=True)
    d = {k: to_dev(v) for k, v in _inputs(1000, seed=120).items()}
    full = _run(d)
    for lo, hi in ((0, 1), (5, 6), (999, 1000), (17, 50), (300, 1000)):
        part = _run(dict(d, out=d["out"][lo:hi].contiguous(), d_lat=d["d_lat"][lo:hi].contiguous()))
        for k in ("latent", "d_out"):
            assert same_bytes(full[k][lo:hi], part[k]), (lo, hi, k)


def test_proj_out_param_grads_zero_padding(gpu_lib):
    """dWp and dbp of 600 tokens equal those of 1100 tokens whose last 500 have
    d_lat = 0, byte for byte (the last chunk grows, a zero chunk is added)."""
    print("[proj_out] zero padding", flush=True)
    d = {k: to_dev(v) for k, v in _inputs(1100, seed=121).items()}
    base = _run(dict(d, out=d["out"][:600].contiguous(), d_lat=d["d_lat"][:600].contiguous()))
    padded = dict(d, d_lat=d["d_lat"].clone())
    padded["d_lat"][600:] = 0
    r = _run(padded)
    assert same_bytes(r["dW"], base["dW"]) and same_bytes(r["db"], base["db"])


def test_proj_out_shapes_through_ops(gpu_lib):
    """[B, S, 3072] tensors: the wrapper flattens tokens; rows equal the flat call."""
    print("[proj_out] batched shapes", flush=True)
    d = {k: to_dev(v) for k, v in _inputs(2 * 300, seed=122).items()}
    from invariant_silu_amd import ops
    x3 = d["out"].view(2, 300, K)
    lat3 = ops.proj_out_fwd(x3, d["W"], d["bias"])
    d3, dW3, db3 = ops.proj_out_bwd(d["d_lat"].view(2, 300, O), x3, d["W"])
    flat = _run(d)
    assert lat3.shape == (2, 300, O) and same_bytes(lat3.reshape(600, O), flat["latent"])
    assert same_bytes(d3.reshape(600, K), flat["d_out"])
    assert same_bytes(dW3, flat["dW"]) and same_bytes(db3, flat["db"])


def test_proj_out_autograd_composes_with_final_modulation(gpu_lib):
    """The final layer as autograd ops (adaln_final, then proj_out): the
    gradients equal the entry points called by hand, byte for byte."""
    print("[proj_out] autograd", flush=True)
    from invariant_silu_amd import ops
    from synthetic_inputs import make_inputs
    inp = make_inputs(2, 40, seed=123)
    d = {k: to_dev(inp[k]) for k in ("x", "temb", "W", "bias")}
    po_in = _inputs(80, seed=124)
    Wp, bp = to_dev(po_in["W"]), to_dev(po_in["bias"])
    d_lat = to_dev(po_in["d_lat"]).view(2, 40, O)
    leaves = {k: v.clone().requires_grad_(True) for k, v in d.items()}
    Wp_l, bp_l = Wp.clone().requires_grad_(True), bp.clone().requires_grad_(True)
    out = ops.adaln_final(leaves["x"], leaves["temb"], leaves["W"], leaves["bias"])
    latent = ops.proj_out(out, Wp_l, bp_l)
    latent.backward(d_lat)
    # by hand
    out2, emb, mean, rstd = ops.fwd(d["x"], d["temb"], d["W"], d["bias"])
    lat2 = ops.proj_out_fwd(out2, Wp, bp)
    d_out, dWp, dbp = ops.proj_out_bwd(d_lat, out2, Wp)
    dx, d_emb, dW, db, dtemb = ops.bwd(d_out, d["x"], mean, rstd, emb, d["temb"], d["W"])
    assert same_bytes(latent.detach(), lat2)
    assert same_bytes(Wp_l.grad, dWp) and same_bytes(bp_l.grad, dbp)
    assert same_bytes(leaves["x"].grad, dx) and same_bytes(leaves["temb"].grad, dtemb)
    assert same_bytes(leaves["W"].grad, dW) and same_bytes(leaves["bias"].grad, db)
