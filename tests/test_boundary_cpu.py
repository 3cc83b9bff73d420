"""CPU-side checks of the C ABI: the library loads, exports every function the
header declares, the binding declares the same names, workspace sizes follow
the documented formulas, and argument validation answers before any device
work (no kernel runs here: there is no GPU in this environment)."""

from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from invariant_silu_amd import lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adaln.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(lib.LIB_PATH):
        pytest.skip("libadaln.so not built (run __graft_entry__.build())")
    return lib.load()


def test_header_declares_the_entry_points():
    names = _declared()
    for fn in ("adaln_proj_fwd", "adaln_proj_bwd", "adaln_norm_mod_fwd", "adaln_norm_mod_bwd",
               "token_tree_sum"):
        assert fn in names
    assert names == set(lib.EXPORTS), names ^ set(lib.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_abi_version_and_strerror(L):
    assert L.adaln_abi_version() == 17 == lib.ABI_VERSION
    header = open(HEADER).read()
    assert re.search(r"#define ADALN_ABI_VERSION (\d+)", header).group(1) == "17"
    for code in range(-8, 1):
        assert len(lib.strerror(code)) >= 2


def test_workspace_sizes(L):
    pad = lambda n: (n + 255) // 256 * 256   # noqa: E731
    for B, S in [(1, 31), (2, 1024), (1, 4096), (64, 1024), (3, 6889), (5, 33), (8, 1024), (9, 3), (17, 2),
                 (65, 2), (128, 3), (129, 3), (300, 1)]:
        T0 = math.ceil(S / 32)
        assert lib.workspace_bytes(lib.OP_NORM_MOD_BWD, B, S, 3072) == pad(B * T0 * 6144 * 8)
        assert lib.workspace_bytes(lib.OP_TOKEN_TREE_SUM, B, S, 100) == pad(B * T0 * 128 * 8)
        # da leaf runs on the matrix cores: 8 for one row of 16 samples, 4 up to
        # four rows, 2 beyond; each run's subtree is 96 column blocks x 2 tiles
        # x 64 lanes x 4 fp64 per row of samples
        rows = math.ceil(B / 16)
        runs = 8 if rows == 1 else 4 if rows <= 4 else 2
        parts = rows * 96 * runs * 2 * 64 * 32
        # B <= 6: 32 fp64 da subtrees per sample and column; B > 6: the SiLU
        # activations, then the run subtrees
        proj_bwd = pad(32 * B * 3072 * 8) if B <= 6 else pad(B * 3072 * 2) + pad(parts)
        assert lib.workspace_bytes(lib.OP_PROJ_BWD, B, S, 3072) == proj_bwd
        assert lib.workspace_bytes(lib.OP_PROJ_FWD, B, S, 3072) == pad(B * 3072 * 2)
        # fp32: the activations, then the fp64 da subtrees (B <= 4) or run subtrees
        sub = pad(32 * B * 3072 * 8) if B <= 4 else pad(parts)
        assert lib.workspace_bytes(lib.OP_BWD_F32, B, S, 3072) == pad(B * T0 * 6144 * 8) + pad(B * 3072 * 4) + sub
        assert lib.workspace_bytes(lib.OP_RESIDUAL_BWD, B, S, 3072) == pad(B * T0 * 9216 * 8)
        C = math.ceil(B * S / 512)
        # proj_out: fp64 dWp / dbp partial sums of 512-token chunks; the forward keeps its partials on chip
        assert lib.workspace_bytes(lib.OP_PROJ_OUT_BWD, B, S, 3072) == pad(C * 64 * 3072 * 8) + pad(C * 64 * 8)
        assert lib.workspace_bytes(lib.OP_PROJ_OUT_FWD, B, S, 3072) == 256
        assert lib.workspace_bytes(lib.OP_FWD_PROJ_OUT, B, S, 3072) == pad(B * 3072 * 2) + 256
    # proj_out: a flat token count beyond the modulation's sequence limit
    T = 1 << 22
    assert lib.workspace_bytes(lib.OP_PROJ_OUT_FWD, 1, T, 3072) == 256
    assert lib.workspace_bytes(lib.OP_PROJ_OUT_BWD, 1, T, 3072) == pad((T // 512) * 64 * 3072 * 8) + pad((T // 512) * 64 * 8)
    assert lib.workspace_bytes(lib.OP_PROJ_OUT_FWD, 1, 65535 * 512 + 1, 3072) == 0
    assert lib.workspace_bytes(lib.OP_NORM_MOD_BWD, 1, 10, 1024) == 0
    assert lib.workspace_bytes(99, 1, 10, 3072) == 0
    assert lib.workspace_bytes(lib.OP_PROJ_BWD, 0, 1, 3072) == 0
    assert lib.workspace_bytes(99, 1, 1, 3072) == 0


def test_validation_before_device_work(L):
    """NULL pointers and bad shapes are reported without touching a device."""
    assert L.adaln_proj_fwd(None, None, None, None, None, 0, 1, 3072, 6144, None) == lib.ERR_NULL
    p = 4096   # a fake, aligned, non-null address: shape checks come first
    assert L.adaln_proj_fwd(p, p, p, p, p, 1 << 20, 1, 1024, 6144, None) == lib.ERR_SHAPE
    # fp32 storage entry points: the same checks, fp32 sizes
    assert L.adaln_fwd_f32(None, p, p, p, p, p, p, p, 1, 4, 3072, 1e-6, None) == lib.ERR_NULL
    assert L.adaln_fwd_f32(p, p, p, p, p, p, p, p, 1, 4, 1024, 1e-6, None) == lib.ERR_SHAPE
    assert L.adaln_fwd_f32(p + 8, p, p, p, p, p, p, p, 1, 4, 3072, 1e-6, None) == lib.ERR_ALIGN
    bufs = [p + (k << 28) for k in range(13)]
    assert L.adaln_bwd_f32(*bufs, 16, 2, 64, 3072, None) == lib.ERR_WORKSPACE
    assert L.adaln_bwd_f32(*bufs[:12], None, 1 << 20, 2, 64, 3072, None) == lib.ERR_NULL
    # residual norm site
    assert L.adaln_residual_fwd(None, p, p, p, p, p, p, 1, 4, 3072, 1e-6, None) == lib.ERR_NULL
    assert L.adaln_residual_fwd(p, p, p, p, p, p, p, 1, 0, 3072, 1e-6, None) == lib.ERR_SHAPE
    rb = [p + (k << 28) for k in range(11)]
    assert L.adaln_residual_bwd(*rb, 16, 2, 64, 3072, None) == lib.ERR_WORKSPACE
    # a workspace smaller than adaln_workspace_bytes(PROJ_FWD) is refused
    assert L.adaln_proj_fwd(p, p + (1 << 20), p + (2 << 20), p + (3 << 20), p + (4 << 20), 16,
                            8, 3072, 6144, None) == lib.ERR_WORKSPACE
    # projection widths: 6144 (final modulation) and 18432 (a block's 6-way
    # modulation) pass the shape check, others do not
    for n in (3072, 12288, 18431, 24576):
        assert L.adaln_proj_fwd(p, p, p, p, p, 1 << 20, 1, 3072, n, None) == lib.ERR_SHAPE
        assert L.adaln_proj_bwd(p, p, p, p, p, p, p, 1 << 20, 1, 3072, n, None) == lib.ERR_SHAPE
    assert L.adaln_proj_fwd(p, p + (1 << 20), p + (2 << 20), p + (3 << 20), p + (4 << 20), 16,
                            8, 3072, 18432, None) == lib.ERR_WORKSPACE
    pb = [p + (k << 28) for k in range(7)]
    assert L.adaln_proj_bwd(*pb, 16, 8, 3072, 18432, None) == lib.ERR_WORKSPACE
    # adaln_proj_bwd_acc: the fp32 outputs are optional (NULL accepted), checked
    # for alignment and for overlap with every input, output and the workspace
    pa = [p + (k << 28) for k in range(10)]   # d_emb temb W dW db dtemb dW32 db32 dtemb32 ws
    assert L.adaln_proj_bwd_acc(*pa[:6], None, None, None, pa[9], 16, 8, 3072, 6144, None) == lib.ERR_WORKSPACE
    assert L.adaln_proj_bwd_acc(*pa[:6], pa[6] + 4, None, None, pa[9], 1 << 30, 8, 3072, 6144,
                                None) == lib.ERR_ALIGN
    assert L.adaln_proj_bwd_acc(*pa[:6], None, None, pa[8] + 8, pa[9], 1 << 30, 8, 3072, 6144,
                                None) == lib.ERR_ALIGN
    assert L.adaln_proj_bwd_acc(*pa[:6], pa[2] + (16 << 20), None, None, pa[9], 1 << 30, 8, 3072, 6144,
                                None) == lib.ERR_OVERLAP            # dW_f32 inside W
    assert L.adaln_proj_bwd_acc(*pa[:6], None, pa[3], None, pa[9], 1 << 30, 8, 3072, 6144,
                                None) == lib.ERR_OVERLAP            # db_f32 on dW
    assert L.adaln_proj_bwd_acc(*pa[:6], None, None, pa[9], pa[9], 1 << 30, 8, 3072, 6144,
                                None) == lib.ERR_OVERLAP            # dtemb_f32 on the workspace
    assert L.adaln_proj_bwd_acc(*pa[:9], pa[9], 1 << 30, 8, 3072, 12288, None) == lib.ERR_SHAPE
    assert L.adaln_proj_bwd_acc(*pa[:5], None, *pa[6:], 1 << 30, 8, 3072, 6144, None) == lib.ERR_NULL
    # the overlap check spans N rows of W: emb 100 MB past W's start lies inside
    # a 6-way W (113 MB) but not inside a final-modulation W (37.7 MB)
    args = (p, p + (1 << 20), p + (200 << 20), p + (101 << 20), p + (300 << 20), 1 << 20, 1, 3072)
    assert L.adaln_proj_fwd(*args, 18432, None) == lib.ERR_OVERLAP
    assert L.adaln_proj_fwd(*args, 6144, None) != lib.ERR_OVERLAP
    # proj_out: T tokens, K = 3072, O = 64; the workspaces hold partial sums
    assert L.adaln_proj_out_fwd(None, p, p, p, p, 1 << 20, 4, 3072, 64, None) == lib.ERR_NULL
    for T, K, O in ((0, 3072, 64), (65535 * 512 + 1, 3072, 64), (4, 3071, 64), (4, 3072, 32)):
        assert L.adaln_proj_out_fwd(p, p, p, p, p, 1 << 30, T, K, O, None) == lib.ERR_SHAPE
        assert L.adaln_proj_out_bwd(p, p, p, p, p, p, p, 1 << 30, T, K, O, None) == lib.ERR_SHAPE
    assert L.adaln_proj_out_fwd(p + 4, p, p, p, p, 1 << 20, 4, 3072, 64, None) == lib.ERR_ALIGN
    po = [p + (k << 28) for k in range(7)]
    assert L.adaln_proj_out_fwd(*po[:5], 255, 1000, 3072, 64, None) == lib.ERR_WORKSPACE
    need = lib.workspace_bytes(lib.OP_PROJ_OUT_BWD, 1, 1000, 3072)
    assert L.adaln_proj_out_bwd(*po, need - 1, 1000, 3072, 64, None) == lib.ERR_WORKSPACE
    # latent overlapping out is caught before the device check
    assert L.adaln_proj_out_fwd(p, p + (1 << 20), p + (2 << 20), p + 6144 * 3, p + (3 << 20), 1 << 20, 8, 3072, 64,
                                None) == lib.ERR_OVERLAP
    # serving forward of the final layer: the modulation's limits on B and S
    fb = [p + (k << 28) for k in range(11)]
    assert L.adaln_fwd_proj_out(*fb[:10], None, 1 << 30, 1, 64, 3072, 64, 1e-6, None) == lib.ERR_NULL
    for B, S, D, O, eps in ((0, 4, 3072, 64, 1e-6), (1, 0, 3072, 64, 1e-6), (1, 4, 1024, 64, 1e-6),
                            (1, 4, 3072, 32, 1e-6), (1, 4, 3072, 64, -1.0), (1, 4, 3072, 64, float("inf"))):
        assert L.adaln_fwd_proj_out(*fb, 1 << 30, B, S, D, O, eps, None) == lib.ERR_SHAPE
    assert lib.workspace_bytes(lib.OP_FWD_PROJ_OUT, 1, 1 << 22, 3072) == 0    # beyond the sequence limit
    assert L.adaln_fwd_proj_out(*fb[:10], p + 8, 1 << 30, 1, 64, 3072, 64, 1e-6, None) == lib.ERR_ALIGN
    need = lib.workspace_bytes(lib.OP_FWD_PROJ_OUT, 6, 64, 3072)
    assert L.adaln_fwd_proj_out(*fb, need - 1, 6, 64, 3072, 64, 1e-6, None) == lib.ERR_WORKSPACE
    # latent over x, and the workspace over mean, are refused before the device check
    over = list(fb)
    over[7] = fb[3] + 4096
    assert L.adaln_fwd_proj_out(*over, need, 6, 64, 3072, 64, 1e-6, None) == lib.ERR_OVERLAP
    over = list(fb)
    over[10] = fb[8]
    assert L.adaln_fwd_proj_out(*over, need, 6, 64, 3072, 64, 1e-6, None) == lib.ERR_OVERLAP
    assert L.adaln_norm_mod_fwd(p, p, p, p, p, 1, 0, 3072, 1e-6, None) == lib.ERR_SHAPE
    assert L.token_tree_sum(p, p, p, 1 << 20, 1, 1, 0, None) == lib.ERR_SHAPE
    # token_tree_fold sizes the caller's pair buffer before reading it
    pairs = lib.workspace_bytes(lib.OP_NORM_MOD_BWD, 2, 4096, 3072)
    assert L.token_tree_fold(p, pairs - 1, p + (1 << 28), 2, 128, 6144, None) == lib.ERR_WORKSPACE
    assert L.token_tree_fold(p, pairs, p + (1 << 28), 2, 128, 6144, None) not in (
        lib.ERR_NULL, lib.ERR_SHAPE, lib.ERR_ALIGN, lib.ERR_WORKSPACE, lib.ERR_OVERLAP)
    assert L.token_tree_fold(p, 1 << 30, p + (1 << 28), 2, 0, 6144, None) == lib.ERR_SHAPE
    assert L.adaln_norm_mod_fwd(p + 2, p, p, p, p, 1, 1, 3072, 1e-6, None) == lib.ERR_ALIGN
    # overlapping output and input is caught before the device check
    assert L.adaln_norm_mod_fwd(p, p + (1 << 20), p, p + (2 << 20), p + (3 << 20), 1, 4, 3072, 1e-6,
                                None) == lib.ERR_OVERLAP


def test_missing_library_fails_loudly(tmp_path):
    saved = lib._lib
    lib._lib = None
    try:
        with pytest.raises(ImportError):
            lib.load(str(tmp_path / "missing.so"))
    finally:
        lib._lib = saved


def test_site_views_validation(L):
    """adaln_site_fwd / _bwd: NULL rules of the two forms, view strides, and the
    row-by-row overlap check of interleaved gradient views (chunks of one
    6-way gradient pass; views whose rows share bytes do not)."""
    p = 4096
    M = 1 << 28
    B, S, D = 4, 64, 3072
    # forward: plain form needs no gate / h; the residual form needs both
    assert L.adaln_site_fwd(p, None, p + M, p + 2 * M, None, 6 * D, None, p + 3 * M, p + 4 * M, p + 5 * M,
                            B, S, D, 1e-6, None) not in (lib.ERR_NULL, lib.ERR_SHAPE, lib.ERR_ALIGN, lib.ERR_OVERLAP)
    assert L.adaln_site_fwd(p, p + 6 * M, p + M, p + 2 * M, None, 6 * D, p + 7 * M, p + 3 * M, p + 4 * M, p + 5 * M,
                            B, S, D, 1e-6, None) == lib.ERR_NULL
    for ld in (D - 8, 6 * D + 4):
        assert L.adaln_site_fwd(p, None, p + M, p + 2 * M, None, ld, None, p + 3 * M, p + 4 * M, p + 5 * M,
                                B, S, D, 1e-6, None) == lib.ERR_SHAPE
    # backward, residual form: gradient views into one [B, 6D] fp32 tensor
    ws = lib.workspace_bytes(lib.OP_RESIDUAL_BWD, B, S, D)
    dm = p + 9 * M

    def bwd(d_shift, d_scale, d_gate, dld):
        return L.adaln_site_bwd(p, p + M, p + 2 * M, p + 3 * M, p + 4 * M, p + 5 * M, p + 6 * M, p + 6 * M + 2 * D,
                                6 * D, p + 7 * M, p + 8 * M, d_shift, d_scale, d_gate, dld, p + 10 * M, ws, B, S, D,
                                None)

    ok = bwd(dm + 4 * 3 * D, dm + 4 * 4 * D, dm + 4 * 2 * D, 6 * D)      # chunks 3, 4, 2
    assert ok not in (lib.ERR_NULL, lib.ERR_SHAPE, lib.ERR_ALIGN, lib.ERR_OVERLAP, lib.ERR_WORKSPACE)
    assert bwd(dm, dm + 4 * (D // 2), dm + 4 * 2 * D, 6 * D) == lib.ERR_OVERLAP   # rows share bytes
    assert bwd(dm, dm + 4 * 6 * D, dm + 4 * 2 * D, 6 * D) == lib.ERR_OVERLAP      # row b of one = row b+1 of the other
    assert bwd(dm, dm + 4 * D, dm + 4 * 2 * D, D) == lib.ERR_OVERLAP               # stride D: rows run into each other
    assert bwd(dm, dm + 4 * D, None, 6 * D) == lib.ERR_NULL                        # residual form needs d_gate
    # plain form: no g_h, h, gate, d_residual, d_gate
    assert L.adaln_site_bwd(p, None, p + 2 * M, None, p + 4 * M, p + 5 * M, p + 6 * M, None, 6 * D, None, p + 8 * M,
                            dm, dm + 4 * D, None, 6 * D, p + 10 * M, ws, B, S, D, None) not in (
        lib.ERR_NULL, lib.ERR_SHAPE, lib.ERR_ALIGN, lib.ERR_OVERLAP, lib.ERR_WORKSPACE)
