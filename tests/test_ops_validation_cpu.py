"""The PyTorch wrappers check every tensor extent the C ABI assumes before
anything reaches it: the library sees pointers only, so a tensor of the wrong
shape would otherwise be read or written out of bounds.  Meta tensors carry
shapes without memory, so these checks run without a GPU; each call must stop
at the shape check (ValueError), never at the later device check."""

from __future__ import annotations

import pytest
import torch

from invariant_silu_amd import ops

D, N, N6 = 3072, 6144, 18432
bf, f32 = torch.bfloat16, torch.float32


def t(*shape, dtype=bf):
    return torch.empty(shape, dtype=dtype, device="meta")


def shape_error(fn, *args, **kw):
    with pytest.raises(ValueError, match="shape|dimensions|needs|d_views"):
        fn(*args, **kw)


def test_wrappers_accept_consistent_shapes_up_to_the_device_check():
    # right shapes on a non-GPU device: the device check is what stops them
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.bwd(t(2, 5, D), t(2, 5, D), t(2, 5, dtype=f32), t(2, 5, dtype=f32), t(2, N), t(2, D), t(N, D))
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.proj_bwd(t(3, N6, dtype=f32), t(3, D), t(N6, D))


def test_projection_shapes():
    shape_error(ops.proj_fwd, t(2, D), t(N + 64, D), t(N + 64))      # unsupported width
    shape_error(ops.proj_fwd, t(2, D), t(N, D), t(N6))               # bias of another width
    shape_error(ops.proj_fwd, t(2, D - 8), t(N, D), t(N))
    shape_error(ops.proj_fwd, t(D), t(N, D), t(N))                   # temb without a batch dim
    shape_error(ops.proj_bwd, t(2, N, dtype=f32), t(2, D), t(N6, D))  # d_emb of the 2-way width, 6-way W
    shape_error(ops.proj_bwd, t(3, N, dtype=f32), t(2, D), t(N, D))   # d_emb batch != temb batch


def test_norm_shapes():
    shape_error(ops.norm_mod_fwd, t(2, 7, D), t(1, N))
    shape_error(ops.norm_mod_fwd, t(2, 7, 1024), t(2, N))
    shape_error(ops.norm_mod_fwd, t(14, D), t(2, N))
    x = t(2, 7, D)
    shape_error(ops.norm_mod_bwd, t(2, 8, D), x, t(2, 7, dtype=f32), t(2, 7, dtype=f32), t(2, N))
    shape_error(ops.norm_mod_bwd, t(2, 7, D), x, t(2, 6, dtype=f32), t(2, 7, dtype=f32), t(2, N))
    shape_error(ops.norm_mod_bwd, t(2, 7, D), x, t(2, 7, dtype=f32), t(14, dtype=f32), t(2, N))
    shape_error(ops.token_tree_sum, t(7, D, dtype=f32))


def test_one_call_shapes():
    x, st = t(2, 7, D), t(2, 7, dtype=f32)
    shape_error(ops.fwd, x, t(1, D), t(N, D), t(N))
    shape_error(ops.fwd, x, t(2, D), t(N6, D), t(N6))                # the one-call path is 2-way only
    shape_error(ops.fwd, x, t(2, D), t(N, D), t(N - 1))
    shape_error(ops.bwd, t(2, 7, D), x, st, st, t(2, N), t(2, D), t(N6, D))
    shape_error(ops.bwd, t(2, 7, D), x, st, st, t(2, N6), t(2, D), t(N, D))
    shape_error(ops.bwd, t(2, 7, D), x, st, st, t(2, N), t(3, D), t(N, D))
    shape_error(ops.bwd, t(1, 7, D), x, st, st, t(2, N), t(2, D), t(N, D))


def test_site_and_residual_shapes():
    x, st = t(2, 7, D), t(2, 7, dtype=f32)
    shape_error(ops.residual_fwd, x, t(2, 6, D), t(2, 3 * D))
    shape_error(ops.residual_fwd, x, x, t(2, 2 * D))
    shape_error(ops.residual_bwd, x, x, x, t(2, 7, D - 8), st, st, t(2, 3 * D))
    shape_error(ops.residual_bwd, x, x, x, x, st, st, t(1, 3 * D))
    shape_error(ops.site_fwd, x, t(2, D), t(2, D - 8))
    shape_error(ops.site_fwd, x, t(2, D), t(2, D), residual=x)        # the residual form needs gate
    shape_error(ops.site_bwd, x, x, st, st, t(3, D))
    shape_error(ops.site_bwd, x, x, st, st, t(2, D), g_h=x, h=x)      # ... and gate
    shape_error(ops.site_bwd, x, x, st, st, t(2, D), d_views=[t(2, D, dtype=f32)])
    shape_error(ops.site_bwd, x, x, st, st, t(2, D), d_views=[t(2, D, dtype=f32), t(3, D, dtype=f32)])


def test_proj_out_shapes():
    shape_error(ops.proj_out_fwd, t(5, D - 8), t(64, D), t(64))
    shape_error(ops.proj_out_fwd, t(5, D), t(32, D), t(32))
    shape_error(ops.proj_out_fwd, t(5, D), t(64, D), t(32))
    shape_error(ops.proj_out_bwd, t(5, 63), t(5, D), t(64, D))
    shape_error(ops.proj_out_bwd, t(4, 64), t(5, D), t(64, D))
    shape_error(ops.fwd_proj_out, t(2, 7, D), t(2, D), t(N, D), t(N), t(64, D), t(32))
    shape_error(ops.fwd_proj_out, t(2, 7, D), t(2, D), t(N, D), t(N), t(48, D), t(48))
    shape_error(ops.fwd_proj_out, t(2, 7, D), t(1, D), t(N, D), t(N), t(64, D), t(64))


def test_call_refuses_tensors_on_two_devices():
    """Every wrapper hands its tensors to one helper that refuses a call whose
    tensors sit on different devices (the kernels would otherwise dereference
    another GPU's addresses), before the library is reached."""
    from types import SimpleNamespace

    a = SimpleNamespace(device=torch.device("cuda", 0))
    b = SimpleNamespace(device=torch.device("cuda", 1))
    with pytest.raises(ValueError, match="one GPU"):
        ops._call((a, None, b), "adaln_proj_fwd")
