"""The pages' token-sum cancellation probe through the fused backward.

RL-Kernel pull request 538 ("Results (H100 sm90, head e23c4a97)": cancellation
screen, and the review thread on token_sum.cu): at S = 6032 a column of ones
holding one +2^26 and one -2^26 must sum to exactly 6030 (the earlier plain
32-way tree gave 6020).  Here the column is the upstream gradient g of
adaln_bwd, so the sum is d_shift, produced by the level-0 tiles inside the
LayerNorm backward and the fold, and it then feeds db, dW and dtemb.  The
placements sweep the same tile, neighbouring tiles, first and last token and
the last, partial tile (6016..6031); the probe columns sit at tile-block and
64-column-group edges.

Checks: d_shift = 6030.0 exactly in every probe column of every sample (and
in the oracle); d_emb bit-identical to the CPU model of the pages' tree
wherever the GPU's LayerNorm statistics equal the oracle's; every output
within the parity gates of the whole oracle; the first sample's per-row
outputs the same bytes alone as in the batch.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import adaln, token_tree
from oracle.fpmath import bits_to_f32
from synthetic_inputs import cancellation_tokens, f32_to_bf16_bits, make_inputs
from tests.gpu_helpers import ROW_KEYS, dev_inputs, run_onecall_dev, same_bytes, to_host
from tests.test_gpu_parity import _gates
from tests.test_gpu_tree_and_boundary import POS

pytestmark = pytest.mark.gpu

S = 6032
D = 3072
# one probe column per placement: first / last columns, 64-column group edges,
# 512-column tile-block edges, the middle
COLS = [0, 1, 63, 64, 511, 512, 1000, 1535, 2047, 2048, 2559, 3000, 3070, 3071]
assert len(COLS) == len(POS)


def _probe_inputs(B: int, seed: int) -> dict:
    inp = make_inputs(B, S, seed=seed)
    g = inp["g"].copy()
    for c, (p, q) in zip(COLS, POS):
        col = f32_to_bf16_bits(cancellation_tokens(S, p, q))
        for b in range(B):
            # later samples carry the placement mirrored in time
            g[b, :, c] = col if b % 2 == 0 else col[::-1]
    inp["g"] = g
    return inp


@pytest.mark.parametrize("seed", [0, 127])
def test_cancellation_probe_through_adaln_bwd(gpu_lib, seed):
    B = 2
    print(f"[cancel] adaln_bwd probe B={B} S={S} seed={seed}", flush=True)
    inp = _probe_inputs(B, seed)
    d = dev_inputs(inp)
    dev = run_onecall_dev(d)
    gpu = to_host(dev)

    fwd = adaln.forward(inp, want_abs=True)
    bwd = adaln.backward(inp, fwd, want_abs=True)
    # the pages' value, in the oracle and on the GPU
    d_shift_cols = [D + c for c in COLS]
    assert np.all(bwd["d_emb"][:, d_shift_cols] == np.float32(6030.0))
    assert np.all(gpu["d_emb"][:, d_shift_cols] == np.float32(6030.0)), gpu["d_emb"][:, d_shift_cols]

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
    assert matched >= 1

    # the first sample alone gives the same per-row bytes
    one = {k: (v[:1] if k in ("x", "temb", "g") else v) for k, v in d.items()}
    alone = run_onecall_dev(one)
    for k in ROW_KEYS:
        assert same_bytes(alone[k], dev[k][:1]), k
