"""adaln_norm_mod_bwd_noalloc, the allocation-free LayerNorm backward with the
token-sum tree, against adaln_norm_mod_bwd with a caller workspace.

It runs adaln_norm_mod_bwd's kernels with the workspace (the tree's level-0
pairs) in the library's fixed device array, so dx and d_emb must carry the
same bytes.  Calls follow one another on the same array, each smaller than
the one before, so a call that read what the previous one left behind would
show.  Sizes whose pairs exceed the array are refused before anything is
launched.
"""

from __future__ import annotations

import ctypes

import pytest
import torch

from invariant_silu_amd import lib, ops
from synthetic_inputs import make_inputs
from tests.gpu_helpers import dev_inputs, same_bytes

pytestmark = pytest.mark.gpu

D = 3072
SCRATCH = 64 << 20


def _noalloc(L):
    fn = L.adaln_norm_mod_bwd_noalloc
    fn.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 3 + [ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def test_noalloc_matches_norm_mod_bwd_on_successive_calls(gpu_lib):
    fn = _noalloc(gpu_lib)
    for B, S, seed in ((3, 4096, 3), (2, 1000, 4), (1, 33, 5)):
        print(f"[noalloc] B={B} S={S} seed={seed}", flush=True)
        d = dev_inputs(make_inputs(B, S, seed=seed, outlier_frac=0.01))
        emb = ops.proj_fwd(d["temb"], d["W"], d["bias"])
        _, mean, rstd = ops.norm_mod_fwd(d["x"], emb)
        ref_dx, ref_demb = ops.norm_mod_bwd(d["g"], d["x"], mean, rstd, emb)
        dx = torch.empty_like(d["x"])
        d_emb = torch.empty((B, 2 * D), dtype=torch.float32, device="cuda")
        p = lambda t: t.data_ptr()   # noqa: E731
        rc = fn(p(d["g"]), p(d["x"]), p(mean), p(rstd), p(emb), p(dx), p(d_emb), B, S, D,
                torch.cuda.current_stream().cuda_stream)
        assert rc == lib.OK, lib.strerror(rc)
        torch.cuda.synchronize()
        assert same_bytes(dx, ref_dx), (B, S, "dx")
        assert same_bytes(d_emb, ref_demb), (B, S, "d_emb")


def test_noalloc_refuses_sizes_beyond_its_array(gpu_lib):
    fn = _noalloc(gpu_lib)
    B, S = 1, 1366 * 32      # 1366 tiles of 49152 bytes of level-0 pairs: past 64 MiB
    assert lib.workspace_bytes(lib.OP_NORM_MOD_BWD, B, S, D) > SCRATCH
    assert lib.workspace_bytes(lib.OP_NORM_MOD_BWD, B, 1365 * 32, D) <= SCRATCH
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    assert fn(*([t.data_ptr()] * 7), B, S, D, None) == lib.ERR_SCRATCH
