"""Degenerate inputs through the one-call path, against the oracle.

The method's own degenerate cases: rows of equal values (variance 0, so
rstd = 1 / sqrt(eps) and n = 0: the output is the shift exactly), a token
sequence of one element per sample, an upstream gradient of zeros (every
gradient zero), SiLU inputs of zero and W of zeros (emb = the bias exactly),
and rows spanning a wide range of magnitudes (x scaled by 2^20, g by 2^-20).
Each case runs at S = 31 (one tile per sample: the LayerNorm backward writes
the token sums' roots) and S = 40 (two tiles: the fold), with the parity
gates of test_gpu_parity.py.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import adaln
from synthetic_inputs import f32_to_bf16_bits, make_inputs
from tests.gpu_helpers import dev_inputs, run_onecall_dev, to_host
from tests.test_gpu_parity import _gates

pytestmark = pytest.mark.gpu


def _degenerate(case: str, B: int, S: int) -> dict:
    inp = make_inputs(B, S, seed=31 + S, outlier_frac=0.0)
    if case == "constant_rows":
        vals = np.array([0.0, 0.75, -3.0, 1.0e4, 2.0 ** -20], np.float32)
        x = np.repeat(vals[np.arange(B * S) % len(vals)], 3072).reshape(B, S, 3072)
        inp["x"] = f32_to_bf16_bits(x)
    elif case == "zero_grad":
        inp["g"] = np.zeros_like(inp["g"])
    elif case == "zero_temb":
        inp["temb"] = np.zeros_like(inp["temb"])
    elif case == "zero_W":
        inp["W"] = np.zeros_like(inp["W"])
    elif case == "wide_range":
        rng = np.random.default_rng(5)
        x = inp["x"].astype(np.uint32) << 16
        xf = x.view(np.float32).copy()
        g = (inp["g"].astype(np.uint32) << 16).view(np.float32).copy()
        rows = rng.choice(B * S, max(1, B * S // 4), replace=False)
        xf.reshape(B * S, 3072)[rows] *= np.float32(2.0 ** 20)
        g.reshape(B * S, 3072)[rows[: len(rows) // 2]] *= np.float32(2.0 ** -20)
        inp["x"], inp["g"] = f32_to_bf16_bits(xf), f32_to_bf16_bits(g)
    else:
        raise ValueError(case)
    return inp


CASES = ["constant_rows", "zero_grad", "zero_temb", "zero_W", "wide_range"]


@pytest.mark.parametrize("S", [31, 40])
@pytest.mark.parametrize("case", CASES)
def test_degenerate_inputs_match_the_oracle(gpu_lib, case, S):
    B = 2
    print(f"[degenerate] case={case} B={B} S={S}", flush=True)
    inp = _degenerate(case, B, S)
    gpu = to_host(run_onecall_dev(dev_inputs(inp)))
    fwd = adaln.forward(inp, want_abs=True)
    bwd = adaln.backward(inp, fwd, want_abs=True)
    rep = _gates(inp, gpu, fwd, bwd, {})
    for k, r in rep.items():
        print(f"  {k}: {r}")
    assert all(r["n_fail"] == 0 for r in rep.values()), rep
    if case == "constant_rows":
        # n = 0 exactly: out is the shift, bit for bit
        shift = fwd["emb_bits"][:, 3072:]
        assert (gpu["out"] == shift[:, None, :]).all()
    if case == "zero_grad":
        for k in ("dx", "dW", "db", "dtemb"):
            assert not np.any(gpu[k] & 0x7FFF), k
        assert not np.any(gpu["d_emb"]), "d_emb"
    if case in ("zero_temb", "zero_W"):
        assert (gpu["emb"] == inp["bias"][None, :]).all()
