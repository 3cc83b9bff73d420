"""Seeded synthetic inputs for the AdaLN final-modulation path.

This module only draws data.  It holds none of the operator's arithmetic, so the
CPU oracle (``oracle/``) and the HIP path can both be fed from it without
sharing any computation.

Every tensor is returned as a ``uint16`` array holding bfloat16 bit patterns.
Values are drawn as float32 with NumPy's PCG64 ``default_rng(seed)`` in a fixed
order -- x, temb, W, bias, upstream gradient g, then the outlier rows -- then
scaled by the tensor's standard deviation and rounded to bfloat16 with
round-to-nearest-even on the integer bit pattern.

The workloads mirror the shapes the RL-Kernel pull request 538 ("What" and
"Prior art & reuse decision" sections) measures for Qwen-Image's final image
stream: hidden width 3072, projection 3072 -> 6144, image-token counts
S = 1024 (512x512 images), 4096 (1024x1024 images), 6032 and 6889.  The pages
measured on a trained checkpoint and a recorded 4096-sample workload; neither
is available, so these random draws stand in for them.
"""

from __future__ import annotations

import numpy as np

HIDDEN = 3072           # D = K: hidden width and conditioning width
PROJ = 2 * HIDDEN       # N: (scale | shift)

SIGMA = {"x": 1.0, "temb": 1.0, "W": 0.02, "bias": 0.01, "g": 1.0}

# Named workloads: (B, S, outlier fraction of rows scaled x20).
WORKLOADS = {
    "tiny_s31": dict(B=1, S=31, outlier_frac=0.0),
    "img512_b2_s1024": dict(B=2, S=1024, outlier_frac=0.0),
    "img1024_b1_s4096": dict(B=1, S=4096, outlier_frac=0.01),
    "batch64_s1024": dict(B=64, S=1024, outlier_frac=0.0),
    # one GPU's share of batch64_s1024 split over eight GPUs by samples
    "batch8_s1024": dict(B=8, S=1024, outlier_frac=0.0),
    # ... and over four GPUs
    "batch16_s1024": dict(B=16, S=1024, outlier_frac=0.0),
    # the pages' large conditioning batch: 2048 samples of 3 tokens
    "batch2048_s3": dict(B=2048, S=3, outlier_frac=0.0),
}
# one sample of the headline's distribution at other sequence lengths
# (S = 1024 ... 65536: 512 x 512 to 4096 x 4096 images at 16 pixels per token)
WORKLOADS.update({f"seq_b1_s{S}": dict(B=1, S=S, outlier_frac=0.01) for S in (1024, 2048, 8192, 16384, 32768, 65536)})
SWEEP_S = (32, 33, 6032, 6889)
SWEEP_B = (1, 2, 4)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_inputs(B: int, S: int, seed: int = 0, outlier_frac: float = 0.0,
                D: int = HIDDEN, io: str = "bf16") -> dict:
    """Draw one batch: x [B,S,D], temb [B,D], W [2D,D], bias [2D], g [B,S,D].

    ``outlier_frac`` of each sample's rows (rounded) are multiplied by 20 in
    float32 before the bfloat16 rounding; the row indices are drawn last, per
    sample, without replacement.  With ``io="fp32"`` the same draws are
    returned as float32 arrays, not rounded to bfloat16 (fp32 storage).
    """
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, S, D), dtype=np.float32)
    temb = rng.standard_normal((B, D), dtype=np.float32)
    W = rng.standard_normal((2 * D, D), dtype=np.float32) * np.float32(SIGMA["W"])
    bias = rng.standard_normal((2 * D,), dtype=np.float32) * np.float32(SIGMA["bias"])
    g = rng.standard_normal((B, S, D), dtype=np.float32)
    k = int(round(outlier_frac * S))
    outliers = []
    if k > 0:
        for b in range(B):
            rows = np.sort(rng.choice(S, size=k, replace=False))
            x[b, rows, :] *= np.float32(20.0)
            outliers.append(rows)
    if io == "fp32":
        return {"x": x, "temb": temb, "W": W, "bias": bias, "g": g, "outlier_rows": outliers,
                "B": B, "S": S, "D": D, "seed": seed, "io": "fp32"}
    return {
        "x": f32_to_bf16_bits(x),
        "temb": f32_to_bf16_bits(temb),
        "W": f32_to_bf16_bits(W),
        "bias": f32_to_bf16_bits(bias),
        "g": f32_to_bf16_bits(g),
        "outlier_rows": outliers,
        "B": B, "S": S, "D": D, "seed": seed,
    }


def make_residual_inputs(B: int, S: int, seed: int = 0, D: int = HIDDEN) -> dict:
    """One batch for the residual norm site: x, residual [B,S,D], mod [B,3D] =
    (shift | scale | gate), upstream gradients g_out, g_h [B,S,D]; bf16 bits.

    Draw order x, residual, mod, g_out, g_h; standard normals scaled by 1 (x,
    residual, gradients) and 0.5 (mod), rounded to bfloat16."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, S, D), dtype=np.float32)
    residual = rng.standard_normal((B, S, D), dtype=np.float32)
    mod = rng.standard_normal((B, 3 * D), dtype=np.float32) * np.float32(0.5)
    g_out = rng.standard_normal((B, S, D), dtype=np.float32)
    g_h = rng.standard_normal((B, S, D), dtype=np.float32)
    return {"x": f32_to_bf16_bits(x), "residual": f32_to_bf16_bits(residual), "mod": f32_to_bf16_bits(mod),
            "g_out": f32_to_bf16_bits(g_out), "g_h": f32_to_bf16_bits(g_h), "B": B, "S": S, "D": D,
            "seed": seed}


def make_proj_inputs(B: int, N: int, seed: int = 0, K: int = HIDDEN, d_sigma: float = 8.0) -> dict:
    """One batch for a modulation projection K -> N and its backward: temb
    [B, K], W [N, K], bias [N] as bf16 bits; d_emb [B, N] fp32 (token sums of
    per-token gradients, so several times larger than a token's gradient).

    Draw order temb, W, bias, d_emb; standard normals scaled by 1, 0.02, 0.01
    and d_sigma; the first three rounded to bfloat16."""
    rng = np.random.default_rng(seed)
    temb = rng.standard_normal((B, K), dtype=np.float32)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    bias = rng.standard_normal(N, dtype=np.float32) * np.float32(0.01)
    d_emb = rng.standard_normal((B, N), dtype=np.float32) * np.float32(d_sigma)
    return {"temb": f32_to_bf16_bits(temb), "W": f32_to_bf16_bits(W), "bias": f32_to_bf16_bits(bias),
            "d_emb": d_emb, "B": B, "K": K, "N": N, "seed": seed}


def make_mod6_inputs(B: int, seed: int = 0, K: int = HIDDEN, d_sigma: float = 8.0) -> dict:
    """One batch for a block's 6-way modulation projection (N = 6K): d_emb
    holds the gradients of both norm sites' shift | scale | gate."""
    return make_proj_inputs(B, 6 * K, seed=seed, K=K, d_sigma=d_sigma)


def make_proj_out_inputs(T: int, seed: int = 0, K: int = HIDDEN, O: int = 64) -> dict:
    """One batch for proj_out (K -> O per token): out [T, K], W [O, K], bias [O],
    d_lat [T, O], all bf16 bits.  Draw order out, W, bias, d_lat; standard
    normals scaled by 1 (out: a modulated LayerNorm output), 0.02, 0.01 and 1."""
    rng = np.random.default_rng(seed)
    out = rng.standard_normal((T, K), dtype=np.float32)
    W = rng.standard_normal((O, K), dtype=np.float32) * np.float32(0.02)
    bias = rng.standard_normal(O, dtype=np.float32) * np.float32(0.01)
    d_lat = rng.standard_normal((T, O), dtype=np.float32)
    return {"out": f32_to_bf16_bits(out), "W": f32_to_bf16_bits(W), "bias": f32_to_bf16_bits(bias),
            "d_lat": f32_to_bf16_bits(d_lat), "T": T, "seed": seed}


def make_workload(name: str, seed: int = 0, io: str = "bf16") -> dict:
    w = WORKLOADS[name]
    return make_inputs(w["B"], w["S"], seed=seed, outlier_frac=w["outlier_frac"], io=io)


def cancellation_tokens(S: int, pos_big: int, pos_neg: int, big: float = 2.0 ** 26) -> np.ndarray:
    """Token column for the cancellation probe: ones, one +big and one -big.

    The RL-Kernel pull request 538 review thread and its H100 results section
    describe this input at S = 6032 with big = 2^26; the exact sum is S - 2.
    """
    v = np.ones(S, dtype=np.float32)
    v[pos_big] = np.float32(big)
    v[pos_neg] = np.float32(-big)
    return v
