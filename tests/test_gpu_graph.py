"""The one-call forward and backward captured in a HIP graph (torch's graph
capture drives hipStreamBeginCapture on the current stream).

The entry points enqueue kernels only: no allocation, memset or
synchronization inside a call, so a serving loop can capture a whole step and
replay it.  Each replay runs on new contents of the captured input buffers,
with eager work on the same stream between replays, and must give the bytes of
the eager calls on the same inputs -- on every replay, not just the first.
"""

from __future__ import annotations

import pytest
import torch

from synthetic_inputs import make_inputs
from tests.gpu_helpers import dev_inputs, same_bytes

pytestmark = pytest.mark.gpu

NAMES = ("out", "emb", "mean", "rstd", "dx", "d_emb", "dW", "db", "dtemb")


def _step(d):
    from invariant_silu_amd import ops
    out, emb, mean, rstd = ops.fwd(d["x"], d["temb"], d["W"], d["bias"])
    grads = ops.bwd(d["g"], d["x"], mean, rstd, emb, d["temb"], d["W"])
    return dict(zip(NAMES, (out, emb, mean, rstd) + tuple(grads)))


@pytest.mark.parametrize("B,S", [(1, 31), (2, 96), (9, 40)])
def test_fwd_bwd_replays_in_a_hip_graph(gpu_lib, B, S):
    """S = 31: one tile per sample (roots written by the LayerNorm backward);
    S = 96: the fold; B = 9: the matrix-core projections with their SiLU
    workspace."""
    print(f"[graph] capture fwd+bwd B={B} S={S}", flush=True)
    static = dev_inputs(make_inputs(B, S, seed=100 + B, outlier_frac=0.0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture
        _step(static)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = _step(static)
    for rep, seed in enumerate((7, 8, 9)):
        new = dev_inputs(make_inputs(B, S, seed=seed + B, outlier_frac=0.01))
        for k in static:
            static[k].copy_(new[k])
        graph.replay()
        ref = _step(new)            # eager, same stream, after the replay
        torch.cuda.synchronize()
        for k in NAMES:
            assert same_bytes(captured[k], ref[k]), f"replay {rep}: {k}"
