"""The stage entry points of the LayerNorm backward give adaln_norm_mod_bwd's
bytes: adaln_norm_mod_bwd_dx (dx alone), adaln_norm_mod_bwd_tiles (the level-0
pairs alone) and adaln_norm_mod_bwd_level0 (both in one launch), each followed
where it applies by token_tree_fold for d_emb."""

from __future__ import annotations

import math

import pytest
import torch

from invariant_silu_amd import lib, ops
from synthetic_inputs import make_inputs
from tests.gpu_helpers import dev_inputs, same_bytes

pytestmark = pytest.mark.gpu

D, N = 3072, 6144


@pytest.mark.parametrize("B,S", [(1, 4096), (2, 33), (3, 97), (1, 1)])
def test_stages_equal_the_one_call_backward(gpu_lib, B, S):
    print(f"[stages] B={B} S={S}", flush=True)
    L = gpu_lib
    d = dev_inputs(make_inputs(B, S, seed=B * 31 + S, outlier_frac=0.01))
    emb = ops.proj_fwd(d["temb"], d["W"], d["bias"])
    _, mean, rstd = ops.norm_mod_fwd(d["x"], emb)
    ref_dx, ref_demb = ops.norm_mod_bwd(d["g"], d["x"], mean, rstd, emb)
    st = torch.cuda.current_stream().cuda_stream
    T0 = math.ceil(S / 32)
    need = lib.workspace_bytes(lib.OP_NORM_MOD_BWD, B, S, D)
    p = lambda t: t.data_ptr()   # noqa: E731

    dx = torch.empty_like(d["x"])
    lib.check("dx", L.adaln_norm_mod_bwd_dx(p(d["g"]), p(d["x"]), p(mean), p(rstd), p(emb), p(dx), B, S, D, st))
    part = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib.check("tiles", L.adaln_norm_mod_bwd_tiles(p(d["g"]), p(d["x"]), p(mean), p(rstd), p(part), need, B, S, D,
                                                  st))
    d_emb = torch.empty((B, N), dtype=torch.float32, device="cuda")
    lib.check("fold", L.token_tree_fold(p(part), need, p(d_emb), B, T0, N, st))
    torch.cuda.synchronize()
    assert same_bytes(dx, ref_dx) and same_bytes(d_emb, ref_demb)

    dx2 = torch.empty_like(d["x"])
    part2 = torch.empty(need, dtype=torch.uint8, device="cuda")
    lib.check("level0", L.adaln_norm_mod_bwd_level0(p(d["g"]), p(d["x"]), p(mean), p(rstd), p(emb), p(dx2),
                                                    p(part2), need, B, S, D, None, None, st))
    d_emb2 = torch.empty((B, N), dtype=torch.float32, device="cuda")
    lib.check("fold", L.token_tree_fold(p(part2), need, p(d_emb2), B, T0, N, st))
    torch.cuda.synchronize()
    assert same_bytes(dx2, ref_dx) and same_bytes(d_emb2, ref_demb)
    # the pair buffer is sized before anything is launched
    assert L.adaln_norm_mod_bwd_level0(p(d["g"]), p(d["x"]), p(mean), p(rstd), p(emb), p(dx2), p(part2), need - 1,
                                       B, S, D, None, None, st) == lib.ERR_WORKSPACE
