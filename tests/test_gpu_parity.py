"""Parity of the HIP path with the CPU oracle, through the C ABI.

Per-op gates (identical inputs for both sides, the oracle's inputs never come
from the GPU):
  bf16 outputs  <= 1 ulp from the fp32 oracle, else <= 1 ulp from the fp64 twin;
  fp32 outputs  |gpu - o| <= 1e-5 |o| + 2^-24 A (A = sum of |terms|), else the twin;
  d_emb         additionally bit-identical to the CPU model of the pages' tree
                applied to the oracle's g and g * n, wherever the GPU's LayerNorm
                statistics of that sample match the oracle's bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import adaln, token_tree
from oracle.fpmath import bits_to_f32
from synthetic_inputs import make_inputs
from tests.compare import bf16_gate, f32_gate
from tests.gpu_helpers import dev_inputs, run_onecall_dev, run_path, run_path_dev, same_bytes

pytestmark = pytest.mark.gpu

CASES = {
    # name: (B, S, seed, outlier fraction)
    "tiny_s31": (1, 31, 0, 0.0),
    "s1": (2, 1, 0, 0.0),
    "ragged_b3_s97": (3, 97, 127, 0.05),
    "b2_s33": (2, 33, 2026, 0.0),
    "img512_b2_s1024": (2, 1024, 0, 0.0),
    "img1024_b1_s4096": (1, 4096, 0, 0.01),
    # six samples: the matrix-core forward projection with the vector-unit
    # projection backward at its widest (NB = 6)
    "b6_s40": (6, 40, 7, 0.0),
    # eight samples: both projections on the matrix cores (the leaf runs of
    # da and the dW tiles in one grid)
    "b8_s40": (8, 40, 7, 0.0),
}


def _print_case(name, B, S, seed):
    print(f"[parity] case={name} B={B} S={S} seed={seed}", flush=True)


def _gates(inp, gpu, fwd, bwd, twin_cache):
    """Return {name: report} for every output."""
    def twin():
        if "f" not in twin_cache:
            twin_cache["f"] = adaln.forward(inp, "fp64")
            twin_cache["b"] = adaln.backward(inp, twin_cache["f"], "fp64")
        return twin_cache["f"], twin_cache["b"]

    rep = {}
    for k, src in (("emb", fwd), ("out", fwd), ("dx", bwd), ("dtemb", bwd), ("dW", bwd), ("db", bwd)):
        r = bf16_gate(gpu[k], src[k + "_bits"])
        if r["n_outside_oracle"]:
            tf, tb = twin()
            r = bf16_gate(gpu[k], src[k + "_bits"], (tf if src is fwd else tb)[k + "_bits"])
        rep[k] = r
    x = bits_to_f32(inp["x"]).astype(np.float64)
    D = x.shape[-1]
    A_mean = np.abs(x).sum(-1) / D
    rep["mean"] = f32_gate(gpu["mean"], fwd["mean"], A_mean)
    rep["rstd"] = f32_gate(gpu["rstd"], fwd["rstd"], np.zeros_like(A_mean))
    r = f32_gate(gpu["d_emb"], bwd["d_emb"], bwd["A_d_emb"])
    if r["n_outside_oracle"]:
        r = f32_gate(gpu["d_emb"], bwd["d_emb"], bwd["A_d_emb"], twin()[1]["d_emb"])
    rep["d_emb"] = r
    return rep


@pytest.mark.parametrize("name", list(CASES))
def test_parity_full(gpu_lib, name):
    B, S, seed, outl = CASES[name]
    _print_case(name, B, S, seed)
    inp = make_inputs(B, S, seed=seed, outlier_frac=outl)
    gpu = run_path(inp)
    fwd = adaln.forward(inp, want_abs=True)
    bwd = adaln.backward(inp, fwd, want_abs=True)
    rep = _gates(inp, gpu, fwd, bwd, {})
    for k, r in rep.items():
        print(f"  {k}: {r}")
    assert all(r["n_fail"] == 0 for r in rep.values()), rep

    # d_emb against the CPU model of the pages' tree, bit for bit
    g = bits_to_f32(inp["g"])
    n = fwd["n"]
    tree = np.concatenate([token_tree.tree_sum(g * n), token_tree.tree_sum(g)], axis=1)
    stats_equal = [(gpu["mean"][b].tobytes() == fwd["mean"][b].tobytes() and
                    gpu["rstd"][b].tobytes() == fwd["rstd"][b].tobytes()) for b in range(B)]
    for b in range(B):
        if stats_equal[b]:
            assert gpu["d_emb"][b].tobytes() == tree[b].tobytes(), f"sample {b}"
    assert sum(stats_equal) >= 1, "LayerNorm statistics differ from the oracle in every sample"


# The pages' long-sequence gradient shapes over their three seeds (RL-Kernel
# pull request 538, "Tests": S = 4096 / 6889 / 6032, seeds 0, 127, 2026), one
# and two samples, through the one-call entry points the bench times.
LONG_CASES = [(S, B, seed) for S in (6032, 6889) for B in (1, 2) for seed in (0, 127, 2026)]


@pytest.mark.parametrize("S,B,seed", LONG_CASES)
def test_parity_long_sequences_onecall(gpu_lib, S, B, seed):
    _print_case(f"long_onecall_s{S}", B, S, seed)
    inp = make_inputs(B, S, seed=seed)
    d = dev_inputs(inp)
    from tests.gpu_helpers import to_host
    gpu = to_host(run_onecall_dev(d))
    fwd = adaln.forward(inp, want_abs=True)
    bwd = adaln.backward(inp, fwd, want_abs=True)
    rep = _gates(inp, gpu, fwd, bwd, {})
    for k, r in rep.items():
        print(f"  {k}: {r}")
    assert all(r["n_fail"] == 0 for r in rep.values()), rep
    g = bits_to_f32(inp["g"])
    tree = np.concatenate([token_tree.tree_sum(g * fwd["n"]), token_tree.tree_sum(g)], axis=1)
    matched = 0
    for b in range(B):
        if (gpu["mean"][b].tobytes() == fwd["mean"][b].tobytes() and
                gpu["rstd"][b].tobytes() == fwd["rstd"][b].tobytes()):
            assert gpu["d_emb"][b].tobytes() == tree[b].tobytes(), f"sample {b}"
            matched += 1
    assert matched >= 1, "LayerNorm statistics differ from the oracle in every sample"


def test_parity_large_batch_sampled(gpu_lib):
    """B = 64, S = 1024 (65,536 rows), in the same launch configuration as the
    bench: per-sample outputs of samples 0, 31, 63 against the oracle run on
    each sample alone, and dW / db rows against the batch oracle."""
    B, S = 64, 1024
    print(f"[parity] case=batch64_s1024 B={B} S={S} seed=0", flush=True)
    inp = make_inputs(B, S, seed=0)
    gpu = run_path(inp)
    for b in (0, 31, 63):
        one = {k: (inp[k][b:b + 1] if k in ("x", "temb", "g") else inp[k]) for k in ("x", "temb", "W", "bias", "g")}
        fwd = adaln.forward(one, want_abs=True)
        bwd = adaln.backward(one, fwd, want_abs=True)
        g1 = {k: gpu[k][b:b + 1] for k in ("emb", "out", "mean", "rstd", "dx", "d_emb", "dtemb")}
        for k, src in (("emb", fwd), ("out", fwd), ("dx", bwd), ("dtemb", bwd)):
            r = bf16_gate(g1[k], src[k + "_bits"])
            if r["n_outside_oracle"]:
                tw = adaln.forward(one, "fp64") if src is fwd else adaln.backward(one, adaln.forward(one, "fp64"), "fp64")
                r = bf16_gate(g1[k], src[k + "_bits"], tw[k + "_bits"])
            print(f"  sample {b} {k}: {r}")
            assert r["n_fail"] == 0
        r = f32_gate(g1["d_emb"], bwd["d_emb"], bwd["A_d_emb"])
        print(f"  sample {b} d_emb: {r}")
        assert r["n_fail"] == 0
        assert f32_gate(g1["rstd"], fwd["rstd"], np.zeros_like(fwd["rstd"]))["n_fail"] == 0
    rows = np.array([0, 1, 1000, 3071, 3072, 4097, 6142, 6143])
    stats = adaln.ln_stats(inp)
    dW, db, de = adaln.param_grads_rows(inp, rows, stats=stats)
    rw = bf16_gate(gpu["dW"][rows], dW)
    rb = bf16_gate(gpu["db"][rows], db)
    print(f"  dW rows: {rw}\n  db rows: {rb}")
    assert rw["max_ulp"] <= 1 and rb["max_ulp"] <= 1


@pytest.mark.parametrize("B,S", [(1, 31), (1, 4096), (2, 1024), (3, 4096), (3, 97), (4, 33), (5, 40), (8, 36),
                                 (9, 17), (16, 5), (12, 40), (64, 64), (70, 33)])
def test_onecall_path_matches_separate_calls(gpu_lib, B, S):
    """adaln_fwd / adaln_bwd give the same bytes as the five separate entry
    points on every branch: the forward's projection on the vector units
    (B <= 4; x within 32 MiB read twice, B = 3, S = 4096 once) or the matrix
    cores (B > 4), the backward's on the vector units (B <= 6) or the matrix
    cores (B > 6; with more than one token tile the fold's launch computes
    SiLU(temb) for them, which adaln_proj_bwd does in a launch of its own)."""
    print(f"[parity] one-call vs separate B={B} S={S}", flush=True)
    d = dev_inputs(make_inputs(B, S, seed=B * 1000 + S, outlier_frac=0.01))
    a = run_path_dev(d)
    b = run_onecall_dev(d)
    for k in a:
        assert same_bytes(a[k], b[k]), k
