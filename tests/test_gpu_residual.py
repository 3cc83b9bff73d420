"""Residual norm site (ScaleResidualLayerNormScaleShift) on the GPU: parity with
oracle/residual.py and bytewise batch invariance.  The reading of the operator
(the pages name it with its rounding points, miles_diffusion pull request 108)
is in oracle/residual.py and include/adaln.h."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import residual, token_tree
from oracle.fpmath import bits_to_f32
from synthetic_inputs import make_residual_inputs
from tests.compare import bf16_gate, f32_gate
from tests.gpu_helpers import bf16_bits, same_bytes, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("x", "residual", "mod", "g_out", "g_h")
ROW_KEYS = ("out", "h", "mean", "rstd", "d_residual", "dx", "d_mod")


def _run(d: dict) -> dict:
    from invariant_silu_amd import ops
    out, h, mean, rstd = ops.residual_fwd(d["x"], d["residual"], d["mod"])
    d_res, dx, d_mod = ops.residual_bwd(d["g_out"], d["g_h"], d["x"], h, mean, rstd, d["mod"])
    return dict(out=out, h=h, mean=mean, rstd=rstd, d_residual=d_res, dx=dx, d_mod=d_mod)


def _slice(d: dict, lo: int, hi: int) -> dict:
    return {k: v[lo:hi] for k, v in d.items()}


@pytest.mark.parametrize("B,S", [(1, 31), (2, 64), (1, 100)])
def test_residual_parity(gpu_lib, B, S):
    print(f"[residual] parity B={B} S={S}", flush=True)
    inp = make_residual_inputs(B, S, seed=60 + B * S)
    gpu = _run({k: to_dev(inp[k]) for k in KEYS})
    torch.cuda.synchronize()
    f = residual.residual_forward(inp)
    b = residual.residual_backward(inp, f, want_abs=True)
    f6 = residual.residual_forward(inp, "fp64")
    b6 = residual.residual_backward(inp, f6, "fp64")
    assert np.array_equal(bf16_bits(gpu["h"]), f["h_bits"])
    for k, o, t in (("out", f["out_bits"], f6["out_bits"]), ("d_residual", b["dh_bits"], b6["dh_bits"]),
                    ("dx", b["dx_bits"], b6["dx_bits"])):
        r = bf16_gate(bf16_bits(gpu[k]), o, t)
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k
    assert f32_gate(gpu["rstd"].cpu().numpy(), f["rstd"], np.zeros_like(f["rstd"], dtype=np.float64))["n_fail"] == 0
    r = f32_gate(gpu["d_mod"].cpu().numpy(), b["d_mod"], b["A_d_mod"])
    print(f"  d_mod: {r}")
    assert r["n_fail"] == 0
    # d_shift: the GPU's token tree against the CPU tree model, bit for bit
    want = token_tree.tree_sum(bits_to_f32(inp["g_out"]))
    assert gpu["d_mod"][:, :3072].cpu().numpy().tobytes() == want.tobytes()


@pytest.mark.parametrize("B,S", [(5, 33), (3, 97)])
def test_residual_singleton_vs_batch(gpu_lib, B, S):
    print(f"[residual] invariance B={B} S={S}", flush=True)
    d = {k: to_dev(v) for k, v in make_residual_inputs(B, S, seed=70).items() if k in KEYS}
    full = _run(d)
    for bi in range(B):
        one = _run(_slice(d, bi, bi + 1))
        for k in ROW_KEYS:
            assert same_bytes(full[k][bi:bi + 1], one[k]), f"sample {bi} {k}"


def test_residual_zero_gradient_tokens(gpu_lib):
    """d_mod is unchanged by trailing tokens whose gradients are zero."""
    print("[residual] zero-gradient tokens", flush=True)
    S0, S1 = 40, 40 + 29
    a = make_residual_inputs(2, S0, seed=80)
    bigger = make_residual_inputs(2, S1, seed=81)
    for k in ("x", "residual", "g_out", "g_h"):
        bigger[k][:, :S0] = a[k]
    bigger["g_out"][:, S0:] = 0
    bigger["g_h"][:, S0:] = 0
    bigger["mod"] = a["mod"]
    r0 = _run({k: to_dev(a[k]) for k in KEYS})
    r1 = _run({k: to_dev(bigger[k]) for k in KEYS})
    assert same_bytes(r0["d_mod"], r1["d_mod"])


def test_residual_bench_shape_full(gpu_lib):
    """B = 1, S = 4096 (the bench's shape, its launch configuration): every
    output against the oracle; d_shift against the CPU tree model bit for bit."""
    print("[residual] B=1 S=4096 full", flush=True)
    inp = make_residual_inputs(1, 4096, seed=0)
    gpu = _run({k: to_dev(inp[k]) for k in KEYS})
    torch.cuda.synchronize()
    f = residual.residual_forward(inp)
    b = residual.residual_backward(inp, f, want_abs=True)
    f6 = residual.residual_forward(inp, "fp64")
    b6 = residual.residual_backward(inp, f6, "fp64")
    assert np.array_equal(bf16_bits(gpu["h"]), f["h_bits"])
    for k, o, t in (("out", f["out_bits"], f6["out_bits"]), ("d_residual", b["dh_bits"], b6["dh_bits"]),
                    ("dx", b["dx_bits"], b6["dx_bits"])):
        r = bf16_gate(bf16_bits(gpu[k]), o, t)
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k
    r = f32_gate(gpu["d_mod"].cpu().numpy(), b["d_mod"], b["A_d_mod"])
    print(f"  d_mod: {r}")
    assert r["n_fail"] == 0
    want = token_tree.tree_sum(bits_to_f32(inp["g_out"]))
    assert gpu["d_mod"][:, :3072].cpu().numpy().tobytes() == want.tobytes()
