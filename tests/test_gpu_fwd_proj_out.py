"""The final layer's serving forward (adaln_fwd_proj_out): the final modulation
and proj_out with the modulated output computed on chip, never stored.

Its results must be the bytes of adaln_fwd followed by adaln_proj_out_fwd on
that call's out (latent, emb, mean, rstd), both parity-tested against the
oracle (test_gpu_parity.py, test_gpu_proj_out.py), at any batch and sequence
shape: ragged token groups, 32-token groups holding tokens of several samples
(S < 32 and S not a multiple of 32), the narrow-batch (B <= 4) and matrix-core
(B > 4) projection paths, the 1024 x 1024 image stream and the largest shapes
the entry point accepts.
"""

from __future__ import annotations

import pytest
import torch

from synthetic_inputs import make_inputs, make_proj_out_inputs
from tests.gpu_helpers import same_bytes, to_dev

pytestmark = pytest.mark.gpu

D = 3072


def _params(seed):
    inp = make_inputs(1, 1, seed=seed)
    po = make_proj_out_inputs(1, seed + 1)
    return (to_dev(inp["temb"]), to_dev(inp["W"]), to_dev(inp["bias"]), to_dev(po["W"]), to_dev(po["bias"]))


def _check(x, temb, W, bias, Wp, bp):
    from invariant_silu_amd import ops
    latent, emb, mean, rstd = ops.fwd_proj_out(x, temb, W, bias, Wp, bp)
    out2, emb2, mean2, rstd2 = ops.fwd(x, temb, W, bias)
    lat2 = ops.proj_out_fwd(out2, Wp, bp)
    assert latent.shape == lat2.shape
    for name, a, b in (("latent", latent, lat2), ("emb", emb, emb2), ("mean", mean, mean2), ("rstd", rstd, rstd2)):
        assert same_bytes(a, b), name


@pytest.mark.parametrize("B,S", [(1, 1), (1, 37), (2, 5), (3, 70), (4, 64), (5, 3), (6, 33), (9, 100)])
def test_fused_equals_unfused(gpu_lib, B, S):
    print(f"[fwd_proj_out] B={B} S={S}", flush=True)
    inp = make_inputs(B, S, seed=200 + 7 * B + S)
    temb, W, bias, Wp, bp = _params(201)
    temb = to_dev(inp["temb"])
    _check(to_dev(inp["x"]), temb, W, bias, Wp, bp)


def test_fused_image_stream(gpu_lib):
    """B = 1, S = 4096 (a 1024 x 1024 image's tokens) and B = 2 of them."""
    for B in (1, 2):
        print(f"[fwd_proj_out] B={B} S=4096", flush=True)
        g = torch.Generator(device="cuda").manual_seed(210 + B)
        x = torch.randn((B, 4096, D), device="cuda", generator=g).to(torch.bfloat16)
        temb = (torch.randn((B, D), device="cuda", generator=g) * 2).to(torch.bfloat16)
        _, W, bias, Wp, bp = _params(212)
        _check(x, temb, W, bias, Wp, bp)


def test_fused_largest_shapes(gpu_lib):
    """S = 32 x 65535 with B = 1 (2.1 M tokens in one sample) and B = 65535 with
    S = 1 (every token its own sample)."""
    _, W, bias, Wp, bp = _params(220)
    g = torch.Generator(device="cuda").manual_seed(221)
    for B, S in ((1, 32 * 65535), (65535, 1)):
        print(f"[fwd_proj_out] B={B} S={S}", flush=True)
        x = torch.randn((B, S, D), device="cuda", generator=g).to(torch.bfloat16)
        temb = torch.randn((B, D), device="cuda", generator=g).to(torch.bfloat16)
        _check(x, temb, W, bias, Wp, bp)
        del x, temb
        torch.cuda.empty_cache()
