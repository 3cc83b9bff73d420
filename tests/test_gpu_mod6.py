"""A block's 6-way modulation projection (N = 6 x 3072 = 18432) on the GPU,
through adaln_proj_fwd / adaln_proj_bwd: parity with oracle/modulation.py and
bytewise batch invariance across the vector-unit (forward B <= 4, backward
B <= 6) and matrix-core (beyond) branches.  bf16 outputs are gated at 1 ulp from the fp32 oracle,
else 1 ulp from its fp64 twin (tests/compare.py).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import modulation
from synthetic_inputs import make_mod6_inputs
from tests.compare import bf16_gate
from tests.gpu_helpers import bf16_bits, same_bytes, to_dev

pytestmark = pytest.mark.gpu

K = 3072
N6 = 6 * K


def _dev(inp: dict) -> dict:
    d = {k: to_dev(inp[k]) for k in ("temb", "W", "bias")}
    d["d_emb"] = torch.from_numpy(np.ascontiguousarray(inp["d_emb"])).cuda()
    return d


def _run(d: dict) -> dict:
    from invariant_silu_amd import ops
    emb = ops.proj_fwd(d["temb"], d["W"], d["bias"])
    dW, db, dtemb = ops.proj_bwd(d["d_emb"], d["temb"], d["W"])
    return dict(emb=emb, dW=dW, db=db, dtemb=dtemb)


@pytest.mark.parametrize("B", [1, 6])
def test_mod6_parity(gpu_lib, B):
    print(f"[mod6] parity B={B}", flush=True)
    inp = make_mod6_inputs(B, seed=90 + B)
    gpu = _run(_dev(inp))
    torch.cuda.synchronize()
    f = modulation.mod6_forward(inp, want_abs=True)
    f6 = modulation.mod6_forward(inp, "fp64")
    r = bf16_gate(bf16_bits(gpu["emb"]), f["emb_bits"], f6["emb_bits"])
    print(f"  emb: {r}")
    assert r["n_fail"] == 0

    b = modulation.mod6_backward(inp, f, want_abs=True)
    b6 = modulation.mod6_backward(inp, f6, "fp64")
    for k in ("dtemb", "dW", "db"):
        r = bf16_gate(bf16_bits(gpu[k]), b[k + "_bits"], b6[k + "_bits"])
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k


@pytest.mark.parametrize("B", [9, 33, 130])
def test_mod6_singleton_vs_batch(gpu_lib, B):
    """emb and dtemb rows are the same bytes alone (vector units) and in the
    batch (matrix cores: one, two or four sample tiles per wave in the
    projection)."""
    print(f"[mod6] invariance B={B}", flush=True)
    d = _dev(make_mod6_inputs(B, seed=95))
    full = _run(d)
    for b in range(B):
        one = _run({k: (v[b:b + 1] if k in ("temb", "d_emb") else v) for k, v in d.items()})
        for k in ("emb", "dtemb"):
            assert same_bytes(full[k][b:b + 1], one[k]), f"sample {b} {k}"
    four = _run({k: (v[:4] if k in ("temb", "d_emb") else v) for k, v in d.items()})
    for k in ("emb", "dtemb"):
        assert same_bytes(full[k][:4], four[k]), k


def test_mod6_param_grads_zero_padding(gpu_lib):
    """dW and db of three samples (vector units) equal those of eleven samples
    whose last eight have d_emb = 0 (matrix cores), byte for byte."""
    print("[mod6] zero padding", flush=True)
    d = _dev(make_mod6_inputs(11, seed=97))
    base = _run({k: (v[:3] if k in ("temb", "d_emb") else v) for k, v in d.items()})
    padded = dict(d)
    padded["d_emb"] = d["d_emb"].clone()
    padded["d_emb"][3:] = 0
    r = _run(padded)
    assert same_bytes(r["dW"], base["dW"]) and same_bytes(r["db"], base["db"])


def test_mod6_rows_equal_final_projection(gpu_lib):
    """Rows 0 .. 6143 of the 6-way projection with W6's first 6144 rows equal to
    a final-modulation W give that projection's emb, byte for byte (the row
    order and the per-row sum do not depend on N)."""
    print("[mod6] prefix equals the N = 6144 projection", flush=True)
    from invariant_silu_amd import ops
    for B in (2, 5):
        d = _dev(make_mod6_inputs(B, seed=99))
        e6 = ops.proj_fwd(d["temb"], d["W"], d["bias"])
        e2 = ops.proj_fwd(d["temb"], d["W"][:2 * K].contiguous(), d["bias"][:2 * K].contiguous())
        assert same_bytes(e6[:, :2 * K], e2), B


def test_mod6_large_batch_sampled(gpu_lib):
    """B = 2048 (the pages' large conditioning batch): emb and dtemb of sampled
    samples (each sample on its own in the oracle), dW and db on sampled rows of
    W (a row's sums run over all 2048 samples)."""
    B = 2048
    print(f"[mod6] B={B} sampled", flush=True)
    inp = make_mod6_inputs(B, seed=98)
    gpu = _run(_dev(inp))
    torch.cuda.synchronize()
    samples = np.array([0, 1, 15, 16, 1023, 2032, 2047])
    sub = dict(inp, temb=inp["temb"][samples], d_emb=inp["d_emb"][samples])
    f, f6 = modulation.mod6_forward(sub), modulation.mod6_forward(sub, "fp64")
    b, b6 = modulation.mod6_backward(sub, f), modulation.mod6_backward(sub, f6, "fp64")
    for k, got, o, t in (("emb", gpu["emb"][samples], f, f6), ("dtemb", gpu["dtemb"][samples], b, b6)):
        r = bf16_gate(bf16_bits(got), o[k + "_bits"], t[k + "_bits"])
        print(f"  {k} (sampled samples): {r}")
        assert r["n_fail"] == 0, k
    rows = np.array([0, 1, 63, 64, 6143, 6144, 9000, 12287, 18367, 18431])
    from oracle import adaln
    W = adaln._val(inp, "W")
    temb = adaln._val(inp, "temb")
    ar, ar6 = adaln.Arith("fp32"), adaln.Arith("fp64")
    # a row of dW and db depends on that row of d_emb and on a of every sample only
    pr = adaln.proj_backward(inp["d_emb"][:, rows], adaln.silu_act(temb, ar), W[rows], temb, ar)
    pr6 = adaln.proj_backward(inp["d_emb"][:, rows], adaln.silu_act(temb, ar6), W[rows], temb, ar6)
    for k, got in (("dW", gpu["dW"][rows]), ("db", gpu["db"][rows])):
        r = bf16_gate(bf16_bits(got), adaln._bits(pr[k]), adaln._bits(pr6[k]))
        print(f"  {k} (sampled rows): {r}")
        assert r["n_fail"] == 0, k
