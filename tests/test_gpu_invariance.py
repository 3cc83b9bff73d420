"""Bytewise batch invariance of the HIP path (GPU against GPU, raw bytes).

The protocol follows RL-Kernel pull request 538, "Prior art & reuse decision":
a singleton against every row of B = 64 / 257 / 2048, dense and boundary batch
sweeps, a 4096-sample workload in 5 chunkings, and B = 2 against B = 1 at
S = 31 / 32 / 33 / 4096 / 6889 / 6032; the pages' seeds 0 / 127 / 2026; plus
repeat determinism and ordered zero-padding of the parameter gradients
("Results": shared-parameter repeat and ordered zero-padding).

Per-sample outputs (emb, out, mean, rstd, dx, d_emb, dtemb) must be the same
bytes whatever the batch; dW and db are batch sums and must be the same bytes
on repeat and with trailing zero-gradient samples appended.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from synthetic_inputs import make_inputs
from tests.gpu_helpers import ROW_KEYS, dev_inputs, run_onecall_dev, run_path_dev, same_bytes

pytestmark = pytest.mark.gpu


def _slice(d: dict, lo: int, hi: int) -> dict:
    return {k: (v[lo:hi] if k in ("x", "temb", "g") else v) for k, v in d.items()}


def _singletons(d: dict, B: int) -> list:
    return [run_path_dev(_slice(d, b, b + 1)) for b in range(B)]


def _assert_rows_equal(batch: dict, singles: list, offset: int = 0, label: str = ""):
    for b, one in enumerate(singles):
        for k in ROW_KEYS:
            assert same_bytes(batch[k][offset + b:offset + b + 1], one[k]), f"{label} sample {b} {k}"


@pytest.mark.parametrize("S", [31, 32, 33, 4096, 6032, 6889])
@pytest.mark.parametrize("seed", [0, 127, 2026])
def test_b2_vs_b1(gpu_lib, S, seed):
    print(f"[invariance] B=2 vs B=1 S={S} seed={seed}", flush=True)
    d = dev_inputs(make_inputs(2, S, seed=seed))
    _assert_rows_equal(run_path_dev(d), _singletons(d, 2), label=f"S={S}")
    # the one-call entry points, batch against singletons of the separate calls
    _assert_rows_equal(run_onecall_dev(d), _singletons(d, 2), label=f"one-call S={S}")


@pytest.mark.parametrize("S", [32, 33, 6032, 6889])
def test_sweep_b4(gpu_lib, S):
    """Odd-length sweep: S in {32, 33, 6032, 6889}, B in {1, 2, 4}."""
    print(f"[invariance] sweep B in (1,2,4) S={S}", flush=True)
    d = dev_inputs(make_inputs(4, S, seed=1))
    singles = _singletons(d, 4)
    for B in (2, 4):
        _assert_rows_equal(run_path_dev(_slice(d, 0, B)), singles[:B], label=f"B={B} S={S}")


def test_singleton_vs_every_row_b64_s1024(gpu_lib):
    print("[invariance] B=64 S=1024 singleton vs every row", flush=True)
    d = dev_inputs(make_inputs(64, 1024, seed=0))
    _assert_rows_equal(run_path_dev(d), _singletons(d, 64), label="B=64")


@pytest.mark.parametrize("B", [257, 2048])
def test_singleton_vs_every_row_large_conditioning_batch(gpu_lib, B):
    """The pages' large-batch shape: S = 3 tokens per sample."""
    print(f"[invariance] B={B} S=3 singleton vs every row", flush=True)
    d = dev_inputs(make_inputs(B, 3, seed=127))
    _assert_rows_equal(run_path_dev(d), _singletons(d, B), label=f"B={B}")


def test_boundary_batch_sweep(gpu_lib):
    sizes = list(range(1, 10)) + [15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
    print(f"[invariance] boundary sweep B in {sizes} S=3", flush=True)
    d = dev_inputs(make_inputs(257, 3, seed=2026))
    singles = _singletons(d, 257)
    for B in sizes:
        _assert_rows_equal(run_path_dev(_slice(d, 0, B)), singles[:B], label=f"B={B}")


def test_chunkings_of_4096_samples(gpu_lib):
    """The 4096-sample workload (S = 3) in 5 chunkings gives identical per-sample bytes."""
    print("[invariance] 4096 samples S=3 in 5 chunkings", flush=True)
    d = dev_inputs(make_inputs(4096, 3, seed=0))
    chunkings = {"1x4096": [4096], "2x2048": [2048] * 2, "64x64": [64] * 64,
                 "4096x1": [1] * 4096, "1000+3000+96": [1000, 3000, 96]}
    ref = None
    for name, parts in chunkings.items():
        outs = {k: [] for k in ROW_KEYS}
        lo = 0
        for n in parts:
            r = run_path_dev(_slice(d, lo, lo + n))
            for k in ROW_KEYS:
                outs[k].append(r[k])
            lo += n
        cat = {k: torch.cat(v, dim=0) for k, v in outs.items()}
        if ref is None:
            ref = cat
        else:
            for k in ROW_KEYS:
                assert same_bytes(cat[k], ref[k]), f"chunking {name} {k}"


def test_repeat_determinism(gpu_lib):
    print("[invariance] repeat determinism B=3 S=1000", flush=True)
    d = dev_inputs(make_inputs(3, 1000, seed=5))
    r1 = run_path_dev(d)
    for _ in range(3):
        r2 = run_path_dev(d)
        for k in r1:
            assert same_bytes(r1[k], r2[k]), k


def test_param_grads_zero_padding(gpu_lib):
    """dW and db are unchanged by trailing samples whose upstream gradient is zero,
    and d_emb is unchanged by trailing zero-gradient tokens."""
    print("[invariance] ordered zero padding", flush=True)
    # 3 samples run the projection backward on the vector units, 11 on the
    # matrix cores
    inp = make_inputs(11, 64, seed=3)
    d = dev_inputs(inp)
    base = run_path_dev(_slice(d, 0, 3))
    padded = dict(d)
    padded["g"] = d["g"].clone()
    padded["g"][3:] = 0
    r = run_path_dev(padded)
    assert same_bytes(r["dW"], base["dW"]) and same_bytes(r["db"], base["db"])
    # trailing zero-gradient tokens
    S2 = 64 + 37
    inp2 = make_inputs(3, S2, seed=3)
    d2 = dev_inputs(inp2)
    d2["x"][:, :64] = d["x"][:3]
    d2["g"][:, :64] = d["g"][:3]
    d2["g"][:, 64:] = 0
    r2 = run_path_dev({"x": d2["x"], "temb": d["temb"][:3], "W": d["W"], "bias": d["bias"], "g": d2["g"]})
    assert same_bytes(r2["d_emb"], base["d_emb"])
    assert same_bytes(r2["dW"], base["dW"]) and same_bytes(r2["db"], base["db"])


def test_projection_paths_agree_on_extreme_inputs(gpu_lib):
    """B <= 4 runs the projection on the vector units and B > 4 on the fp64
    matrix cores; emb must be the same bytes either way.  The inputs reach where
    an fp32 product of the operands would lose bits: SiLU of temb near -90 is a
    bf16 subnormal (or zero), and W spans 2^-40 .. 2^20, so some products lie
    far below fp32's normal range while others dominate the sums."""
    print("[invariance] projection paths, extreme inputs, B=40 vs 1, 4 and 8", flush=True)
    from invariant_silu_amd import ops
    from synthetic_inputs import f32_to_bf16_bits
    from tests.gpu_helpers import to_dev
    rng = np.random.default_rng(11)
    B = 40
    temb = rng.standard_normal((B, 3072), dtype=np.float32)
    mask = rng.random((B, 3072)) < 0.2
    temb[mask] = -rng.uniform(86.0, 98.0, int(mask.sum())).astype(np.float32)
    W = rng.standard_normal((6144, 3072), dtype=np.float32)
    W *= np.exp2(rng.integers(-40, 21, (6144, 3072))).astype(np.float32)
    bias = rng.standard_normal(6144, dtype=np.float32)
    t_d, W_d, b_d = (to_dev(f32_to_bf16_bits(v)) for v in (temb, W, bias))
    emb = ops.proj_fwd(t_d, W_d, b_d)
    assert torch.isfinite(emb.float()).all()
    for b in range(B):
        assert same_bytes(emb[b:b + 1], ops.proj_fwd(t_d[b:b + 1], W_d, b_d)), f"sample {b} (B=1)"
    for lo in range(0, B, 4):
        assert same_bytes(emb[lo:lo + 4], ops.proj_fwd(t_d[lo:lo + 4], W_d, b_d)), f"samples {lo}.. (B=4)"
    for lo in range(0, B, 8):
        assert same_bytes(emb[lo:lo + 8], ops.proj_fwd(t_d[lo:lo + 8], W_d, b_d)), f"samples {lo}.. (B=8)"
