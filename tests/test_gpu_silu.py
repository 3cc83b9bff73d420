"""Exhaustive check of a = bf16(SiLU(temb)) on the GPU against the oracle's
float64 definition, over every finite bf16 input pattern.

The activation is observed through adaln_proj_fwd with W = [I; 0] and b = 0:
emb[:, :D] is then the single exact product a * 1 rounded back to bf16, i.e.
a itself (with -0 becoming +0, on both sides).  The backward's copy of the same
function is checked the same way through dW at B = 1 with d_emb = 1 on row k
(dW[k, :] = bf16(+0 + 1 * a), i.e. a with -0 turned into +0)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from invariant_silu_amd import ops
from oracle import adaln
from tests.gpu_helpers import bf16_bits, to_dev

pytestmark = pytest.mark.gpu
D = 3072


def _all_finite_bf16():
    v = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (v & 0x7F80) != 0x7F80
    v = v[finite]
    pad = (-len(v)) % D
    return np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(-1, D)


def test_silu_exhaustive_forward(gpu_lib):
    temb = _all_finite_bf16()                       # [22, 3072]
    B = temb.shape[0]
    W = np.zeros((2 * D, D), np.uint16)
    W[np.arange(D), np.arange(D)] = 0x3F80          # 1.0
    bias = np.zeros(2 * D, np.uint16)
    emb = bf16_bits(ops.proj_fwd(to_dev(temb), to_dev(W), to_dev(bias)))
    inp = {"x": np.zeros((B, 1, D), np.uint16), "temb": temb, "W": W, "bias": bias}
    a = adaln.silu_act(adaln._val(inp, "temb"), adaln.Arith("fp32"))
    want = adaln.projection(a, adaln._val(inp, "W"), adaln._val(inp, "bias"), adaln.Arith("fp32"))
    from oracle.fpmath import f32_to_bf16_bits
    want_bits = f32_to_bf16_bits(want)
    bad = np.nonzero(emb != want_bits)
    assert bad[0].size == 0, [(hex(int(temb[i, j % D])), hex(int(emb[i, j])), hex(int(want_bits[i, j])))
                              for i, j in zip(*bad)][:10]


def test_silu_exhaustive_backward_copy(gpu_lib):
    """dW[j, k] at B = 1 is bf16(d_emb[j] * a[k]); with d_emb = 1 it is a[k]."""
    temb = _all_finite_bf16()
    rows = []
    W = torch.zeros((2 * D, D), dtype=torch.bfloat16, device="cuda")
    d_emb = torch.zeros((1, 2 * D), dtype=torch.float32, device="cuda")
    d_emb[0, 5] = 1.0
    for b in range(temb.shape[0]):
        dW, db, dtemb = ops.proj_bwd(d_emb, to_dev(temb[b:b + 1]), W)
        rows.append(bf16_bits(dW[5]))
    got = np.stack(rows)
    ar = adaln.Arith("fp32")
    a = adaln.silu_act(adaln._val({"temb": temb}, "temb"), ar)
    from oracle.fpmath import f32_to_bf16_bits
    # dW is a batch sum: one term accumulated from +0 (so -0 becomes +0)
    want = f32_to_bf16_bits(ar.sum([np.asarray(a, np.float32) * np.float32(1.0)], a.shape))
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, [(hex(int(temb[i, j])), hex(int(got[i, j])), hex(int(want[i, j])))
                              for i, j in zip(*bad)][:10]
