"""adaln_proj_bwd_acc on the GPU: the projection backward with the fp32 values
its bf16 outputs are rounded from (dW_f32, db_f32, dtemb_f32).

* the bf16 outputs are the same bytes as adaln_proj_bwd's, and each is the
  bf16 rounding of its fp32 output;
* the fp32 outputs pass the fp32 gate against the oracle's values before
  their storage rounding (dW_acc, db_acc, dtemb_acc), the fp64 twin
  arbitrating, on the vector-unit (B <= 6) and matrix-core (B > 6) paths and
  at both projection widths;
* dtemb_f32 rows are bytewise batch-invariant across the vector-unit path
  and the three matrix-core forms of da (8, 4 or 1 leaf runs per block);
* a NULL fp32 pointer is accepted and changes none of the other outputs.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import adaln
from oracle.fpmath import bits_to_f32
from synthetic_inputs import make_proj_inputs
from tests.compare import f32_gate
from tests.gpu_helpers import same_bytes, to_dev

pytestmark = pytest.mark.gpu

K = 3072
N, N6 = 2 * K, 6 * K


def _case(B: int, N: int, seed: int) -> tuple[dict, dict]:
    """(host, device) inputs of a projection backward K -> N."""
    inp = make_proj_inputs(B, N, seed=seed)
    dev = dict(d_emb=torch.from_numpy(np.ascontiguousarray(inp["d_emb"])).cuda(), temb=to_dev(inp["temb"]),
               W=to_dev(inp["W"]))
    return inp, dev


def _oracle(inp: dict, mode: str) -> dict:
    ar = adaln.Arith(mode)
    temb = bits_to_f32(inp["temb"])
    a = adaln.silu_act(temb, ar)
    return adaln.proj_backward(inp["d_emb"], a, bits_to_f32(inp["W"]), temb, ar, want_abs=(mode == "fp32"))


def _f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


@pytest.mark.parametrize("n,B", [(N, 1), (N, 3), (N, 6), (N, 16), (N, 17), (N, 70), (N6, 1), (N6, 6), (N6, 10),
                                 (N6, 40)])
def test_proj_bwd_acc_parity(gpu_lib, n, B):
    from invariant_silu_amd import ops
    print(f"[proj_bwd_acc] N={n} B={B}", flush=True)
    host, d = _case(B, n, seed=300 + B)
    plain = ops.proj_bwd(d["d_emb"], d["temb"], d["W"])
    acc = ops.proj_bwd(d["d_emb"], d["temb"], d["W"], want_f32=True)
    torch.cuda.synchronize()
    for name, p, q in zip(("dW", "db", "dtemb"), plain, acc[:3]):
        assert same_bytes(p, q), f"{name}: bf16 output differs from adaln_proj_bwd"
    for name, b16, f32 in zip(("dW", "db", "dtemb"), acc[:3], acc[3:]):
        assert same_bytes(b16, f32.to(torch.bfloat16)), f"{name}: bf16 output is not bf16(fp32 output)"

    o = _oracle(host, "fp32")
    t = _oracle(host, "fp64")
    ds = np.abs(np.asarray(adaln.dsilu(bits_to_f32(host["temb"]), adaln.Arith("fp32")), np.float64))
    gates = {
        "dW_f32": f32_gate(_f32(acc[3]), o["dW_acc"], o["A_dW"], t["dW_acc"]),
        "db_f32": f32_gate(_f32(acc[4]), o["db_acc"], o["A_db"], t["db_acc"]),
        # da's rounding scaled by |silu'|, plus the product's own rounding (within REL)
        "dtemb_f32": f32_gate(_f32(acc[5]), o["dtemb_acc"], np.asarray(o["A_da"], np.float64) * ds,
                              t["dtemb_acc"]),
    }
    for k, r in gates.items():
        print(f"  {k}: {r}")
        assert r["n_fail"] == 0, k


@pytest.mark.parametrize("n,B", [(N, 9), (N, 40), (N6, 70)])
def test_proj_bwd_acc_dtemb_batch_invariant(gpu_lib, n, B):
    """dtemb and dtemb_f32 rows are the same bytes alone (vector units), in a
    batch of 9 .. 16 (8 leaf runs per matrix-core block), of 17 .. 64 (4 runs)
    and beyond (one block over all 128 leaves)."""
    from invariant_silu_amd import ops
    print(f"[proj_bwd_acc] invariance N={n} B={B}", flush=True)
    _, d = _case(B, n, seed=321 + B)
    full = ops.proj_bwd(d["d_emb"], d["temb"], d["W"], want_f32=True)
    for b in sorted({0, B // 2, B - 1}):
        one = ops.proj_bwd(d["d_emb"][b:b + 1], d["temb"][b:b + 1], d["W"], want_f32=True)
        assert same_bytes(full[2][b:b + 1], one[2]) and same_bytes(full[5][b:b + 1], one[5]), f"sample {b}"
    for lo, hi in ((B - 9, B), (max(0, B - 16), B), (max(0, B - 40), B)):
        sub = ops.proj_bwd(d["d_emb"][lo:hi], d["temb"][lo:hi], d["W"], want_f32=True)
        assert same_bytes(full[2][lo:hi], sub[2]) and same_bytes(full[5][lo:hi], sub[5]), f"samples {lo}..{hi}"


@pytest.mark.parametrize("B", [2, 7, 11])
def test_proj_bwd_acc_null_outputs(gpu_lib, B):
    """Only dW_f32 requested (db_f32, dtemb_f32 NULL): it and the bf16 outputs
    match the call that asks for all three."""
    from invariant_silu_amd import lib, ops
    print(f"[proj_bwd_acc] NULL outputs B={B}", flush=True)
    _, d = _case(B, N, seed=330 + B)
    ref = ops.proj_bwd(d["d_emb"], d["temb"], d["W"], want_f32=True)
    W, temb, d_emb = d["W"], d["temb"], d["d_emb"]
    n = W.shape[0]
    dW = torch.empty_like(W)
    db = torch.empty((n,), dtype=torch.bfloat16, device=W.device)
    dtemb = torch.empty_like(temb)
    dW32 = torch.empty(W.shape, dtype=torch.float32, device=W.device)
    ws = torch.empty(max(lib.workspace_bytes(lib.OP_PROJ_BWD, B, 1, K), 16), dtype=torch.uint8, device=W.device)
    lib.call("adaln_proj_bwd_acc", d_emb.data_ptr(), temb.data_ptr(), W.data_ptr(), dW.data_ptr(), db.data_ptr(),
             dtemb.data_ptr(), dW32.data_ptr(), None, None, ws.data_ptr(), ws.numel(), B, K, n,
             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert same_bytes(dW32, ref[3])
    assert same_bytes(dW, ref[0]) and same_bytes(db, ref[1]) and same_bytes(dtemb, ref[2])
