"""token_tree_sum on the GPU, and the C-ABI boundary contract on the GPU.

token_tree_sum: the pages' cancellation probe (6030 for every placement of the
+/-2^26 tokens), bit-identity with the CPU model of the tree, zero-padding
neutrality, S = 1 (a fresh output, never a view of the input).

Boundary (RL-Kernel pull request 538 review thread): misaligned views are
copied to aligned storage by the wrapper and give the same bytes as aligned
copies; the C ABI rejects misaligned pointers, overlapping outputs, short
workspaces and bad shapes before launching anything.
"""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from invariant_silu_amd import lib, ops
from oracle import token_tree
from synthetic_inputs import cancellation_tokens, make_inputs
from tests.gpu_helpers import dev_inputs, run_path_dev, same_bytes

pytestmark = pytest.mark.gpu


def test_selftest_passes(gpu_lib):
    assert ops.selftest() == 0


POS = [(0, 32), (0, 1), (5, 6000), (6031, 0), (31, 32), (6016, 6031), (100, 4000), (1, 2),
       (6030, 6031), (3000, 3001), (64, 96), (6015, 6016), (0, 6031), (17, 4113)]


def test_cancellation_probe_gpu(gpu_lib):
    print("[tree] cancellation probe S=6032", flush=True)
    cols = np.stack([cancellation_tokens(6032, p, q) for p, q in POS], axis=1)   # [S, H]
    x = torch.from_numpy(np.stack([cols, cols[:, ::-1].copy()])).cuda()          # [2, S, H]
    out = ops.token_tree_sum(x).cpu().numpy()
    assert np.all(out == np.float32(6030.0)), out


@pytest.mark.parametrize("S", [1, 2, 31, 32, 33, 1000, 1024, 1025, 4096, 6032, 6889, 40000])
def test_tree_matches_cpu_model_bitwise(gpu_lib, S):
    print(f"[tree] vs CPU model S={S}", flush=True)
    rng = np.random.default_rng(S)
    H = 70 if S < 10000 else 17
    x = (rng.standard_normal((3, S, H)) * np.exp2(rng.integers(-12, 12, (3, S, H)))).astype(np.float32)
    got = ops.token_tree_sum(torch.from_numpy(x).cuda()).cpu().numpy()
    want = token_tree.tree_sum(x)
    assert got.tobytes() == want.tobytes()


def test_tree_zero_padding_and_s1(gpu_lib):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((2, 45, 33)).astype(np.float32)
    xp = np.concatenate([x, np.zeros((2, 1000, 33), np.float32)], axis=1)
    a = ops.token_tree_sum(torch.from_numpy(x).cuda())
    b = ops.token_tree_sum(torch.from_numpy(xp).cuda())
    assert same_bytes(a, b)
    one = torch.from_numpy(x[:, :1, :].copy()).cuda()
    r = ops.token_tree_sum(one)
    assert r.data_ptr() != one.data_ptr()
    assert same_bytes(r, one[:, 0, :].contiguous())


def test_misaligned_views_match_aligned_copies(gpu_lib):
    """Inputs viewed at a one-element storage offset (not 16-byte aligned)
    give the same forward and gradient bytes as aligned copies."""
    print("[boundary] misaligned views", flush=True)
    inp = make_inputs(2, 40, seed=4)
    d = dev_inputs(inp)
    ref = run_path_dev(d)
    mis = {}
    for k, v in d.items():
        store = torch.empty(v.numel() + 1, dtype=v.dtype, device=v.device)
        view = store[1:].view(v.shape)
        view.copy_(v)
        assert view.data_ptr() % 16 != 0
        mis[k] = view
    got = run_path_dev(mis)
    for k in ref:
        assert same_bytes(ref[k], got[k]), k


def test_c_abi_rejects_bad_arguments(gpu_lib):
    L = lib.load()
    B, S, D = 1, 40, 3072
    x = torch.zeros((B, S, D), dtype=torch.bfloat16, device="cuda")
    emb = torch.zeros((B, 2 * D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    mean = torch.empty((B, S), dtype=torch.float32, device="cuda")
    rstd = torch.empty_like(mean)
    st = torch.cuda.current_stream().cuda_stream
    p = lambda t: t.data_ptr()   # noqa: E731
    f = L.adaln_norm_mod_fwd
    assert f(p(x), p(emb), p(out), p(mean), p(rstd), B, S, D, 1e-6, st) == lib.OK
    assert f(p(x) + 2, p(emb), p(out), p(mean), p(rstd), B, S, D, 1e-6, st) == lib.ERR_ALIGN
    assert f(p(x), p(emb), p(x), p(mean), p(rstd), B, S, D, 1e-6, st) == lib.ERR_OVERLAP
    assert f(p(x), p(emb), p(out), p(mean), p(mean), B, S, D, 1e-6, st) == lib.ERR_OVERLAP
    assert f(p(x), p(emb), p(out), p(mean), p(rstd), B, S, 1024, 1e-6, st) == lib.ERR_SHAPE
    assert f(p(x), p(emb), p(out), p(mean), p(rstd), 0, S, D, 1e-6, st) == lib.ERR_SHAPE
    assert f(None, p(emb), p(out), p(mean), p(rstd), B, S, D, 1e-6, st) == lib.ERR_NULL
    g = torch.zeros_like(x)
    dx = torch.empty_like(x)
    d_emb = torch.empty((B, 2 * D), dtype=torch.float32, device="cuda")
    need = lib.workspace_bytes(lib.OP_NORM_MOD_BWD, B, S, D)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    fb = L.adaln_norm_mod_bwd
    assert fb(p(g), p(x), p(mean), p(rstd), p(emb), p(dx), p(d_emb), p(ws), need, B, S, D, st) == lib.OK
    assert fb(p(g), p(x), p(mean), p(rstd), p(emb), p(dx), p(d_emb), p(ws), need - 1, B, S, D, st) == lib.ERR_WORKSPACE
    assert fb(p(g), p(x), p(mean), p(rstd), p(emb), p(dx), p(ws), p(ws), need, B, S, D, st) == lib.ERR_OVERLAP
    torch.cuda.synchronize()


def test_autograd_function_matches_direct_calls(gpu_lib):
    inp = make_inputs(2, 50, seed=21)
    d = dev_inputs(inp)
    ref = run_path_dev(d)
    x = d["x"].clone().requires_grad_(True)
    temb = d["temb"].clone().requires_grad_(True)
    W = d["W"].clone().requires_grad_(True)
    b = d["bias"].clone().requires_grad_(True)
    out = ops.adaln_final(x, temb, W, b)
    out.backward(d["g"])
    assert same_bytes(out, ref["out"])
    assert same_bytes(x.grad, ref["dx"])
    assert same_bytes(temb.grad, ref["dtemb"])
    assert same_bytes(W.grad, ref["dW"])
    assert same_bytes(b.grad, ref["db"])
