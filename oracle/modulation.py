"""A transformer block's 6-way modulation projection, written out plainly.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages:
  RL-Kernel pull request 538, "What": the final modulation reuses the
  companion pull request's (537, "AdaLN modulation projection") fixed-order
  projection and its backward unchanged; "Prior art & reuse decision": the
  other library's fused operator takes its scale / shift as views of
  temb.chunk(6, dim=2) at hidden width 3072, i.e. six chunks of one projection
  3072 -> 6 x 3072; "Results": all three streams of the model are revalidated.

Reading (the pages give the width and the chunk count, not the order of the
chunks; this is the plainest one, the same per-site order as
oracle/residual.py):
  emb6 = bf16(SiLU(temb) @ W6^T + b6)             W6 [18432, 3072], b6 [18432]
       = (shift1 | scale1 | gate1 | shift2 | scale2 | gate2)
  chunks 0..2 modulate the block's first norm site, chunks 3..5 its second.
The arithmetic is the final modulation's projection at N = 18432: every
product exact, fp32 accumulation, bias in fp32, one bf16 rounding
(oracle/adaln.py: `projection`, `proj_backward`).  The backward takes the
fp32 gradient of emb6 (both sites' d_shift | d_scale | d_gate) and gives dW6,
db6 and dtemb.

Pins: tests/test_oracle_pins.py (P-22, P-23).
"""

from __future__ import annotations

import numpy as np

from .adaln import Arith, _bits, _val, proj_backward, projection, silu_act

CHUNKS = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")


def mod6_forward(inp: dict, mode: str = "fp32", want_abs: bool = False) -> dict:
    """``inp``: temb [B, K], W [6K, K], bias [6K] as bf16 bit arrays.
    Returns a (the SiLU activations), emb [B, 6K] and, in fp32/fp64 modes,
    emb_bits; with ``want_abs`` also A_emb (sum of |terms|)."""
    ar = Arith(mode)
    temb = _val(inp, "temb")
    a = silu_act(temb, ar)
    r = projection(a, _val(inp, "W"), _val(inp, "bias"), ar, want_abs)
    emb, A = r if want_abs else (r, None)
    out = dict(a=a, emb=emb)
    if mode != "exact":
        out["emb_bits"] = _bits(emb)
    if want_abs:
        out["A_emb"] = A
    return out


def mod6_backward(inp: dict, fwd: dict, mode: str = "fp32", want_abs: bool = False) -> dict:
    """``inp``: d_emb [B, 6K] fp32 values (plus the forward's temb, W).
    Returns da, dtemb, dW, db (and ``*_bits`` of the bf16 outputs; A_da,
    A_dW, A_db with ``want_abs``)."""
    ar = Arith(mode)
    d_emb = np.asarray(inp["d_emb"], dtype=np.float32)
    res = proj_backward(d_emb, fwd["a"], _val(inp, "W"), _val(inp, "temb"), ar, want_abs)
    if mode != "exact":
        res.update(dtemb_bits=_bits(res["dtemb"]), dW_bits=_bits(res["dW"]), db_bits=_bits(res["db"]))
    return res


def site_chunks(emb6: np.ndarray, site: int) -> dict:
    """(shift, scale, gate) of norm site 1 or 2 as column slices of emb6."""
    K = emb6.shape[1] // 6
    base = 3 * (site - 1)
    return {name[:-1]: emb6[:, (base + i) * K:(base + i + 1) * K] for i, name in enumerate(CHUNKS[base:base + 3])}
