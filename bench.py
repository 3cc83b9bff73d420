#!/usr/bin/env python3
"""Throughput of the batch-invariant AdaLN final modulation, forward + backward.

One step is the whole hot path over one batch of synthetic input, through the
C ABI: adaln_fwd (projection and LayerNorm statistics side by side, then the
modulation) and adaln_bwd (dx rows and level-0 token tiles in one launch, the
tree fold, then the projection backward: dW and db, da and dtemb).  Default
workload: one 1024x1024 image stream, B = 1, S = 4096 tokens, D = 3072, bf16
storage, 1% outlier rows x20.  --storage fp32 runs the fp32-storage entry
points (adaln_fwd_f32 / adaln_bwd_f32) on the same draws, unrounded.
--site residual times a block's residual norm site instead (adaln_residual_fwd:
h = residual + gate * x, LayerNorm of h, modulation; adaln_residual_bwd: dh and
dx rows with the level-0 tiles of d_shift / d_scale, the d_gate tiles, the
fold) at the same B and S, bf16 storage.  --site mod6 times a block's 6-way
modulation projection (adaln_proj_fwd and adaln_proj_bwd at N = 18432) at the
workload's B.  --site proj_out times the 3072 -> 64 projection after the final
modulation (adaln_proj_out_fwd and adaln_proj_out_bwd) over the workload's B * S
tokens.  --site serve times the final layer's serving forward
(adaln_fwd_proj_out: the final modulation's projection and statistics, then
proj_out with the modulated output computed on chip) on the final workload.

Measurement (inputs resident in HBM before anything is timed):
  * cold caches, the headline: before the forward and before the backward a
    flush writes and then reads back 768 MiB (three times the 256 MB
    memory-side cache), and HIP events on the step's stream bracket each phase
    (the flushes are outside them); ms_per_step is the mean over the timed
    steps of forward + backward, and at least 100 cold steps give the median,
    p10 and p90;
  * warm, beside it: back-to-back steps over several independent copies of
    every buffer, so no step finds the previous step's data in the cache, but
    the backward finds what the forward of the same step read;
  * the ceiling: a hand-written 16-byte-per-lane streaming copy of the step's
    bytes, after the same flush (libadaln_bench.so, not part of the operator's
    library).

Prints ONE JSON line.  `roofline` covers the dominant kernel, the backward's
first launch (g and x in, dx and the level-0 token tiles out), timed on its
own through adaln_norm_mod_bwd_level0 with events around each launch, after
the same flush as in the step; `cpu_baseline` is the NumPy oracle timed on
this host on the same workload (one thread, and every core on independent
copies), in child processes started before this process touches the GPU.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

D = 3072
N = 2 * D
HBM_PEAK_GBPS = 8000.0
FP64_MFMA_PEAK_TFLOPS = 78.6   # MI355X dense fp64 matrix peak
MALL_BYTES = 256 << 20
MIN_STAT_STEPS = 100   # cold steps behind the median / p10 / p90 (at least)
MIN_KERNEL_LAUNCHES = 20   # timed launches of the dominant kernel (at least)
FLUSH_BYTES = 768 << 20   # written, then read back, before each timed phase (3x the MALL)
METRIC = "fwd+bwd tokens/sec + achieved HBM GB/s at S=4096 D=3072 bf16 (batch-invariant)"
METRIC_RESIDUAL = "residual norm site fwd+bwd tokens/sec at D=3072 bf16 (batch-invariant)"
METRIC_MOD6 = "6-way modulation projection fwd+bwd samples/sec at 3072->18432 bf16 (batch-invariant)"
N6 = 6 * D
PO = 64           # proj_out channels
METRIC_PROJ_OUT = "proj_out fwd+bwd tokens/sec at 3072->64 bf16 (batch-invariant)"
METRIC_SERVE = "final layer serving fwd (modulation + proj_out) tokens/sec at D=3072->64 bf16 (batch-invariant)"


def algorithmic_bytes(B: int, S: int, el: int = 2) -> int:
    """Bytes the method must move per step (no partials, no re-reads), with
    el-byte storage: x read twice, out, g, dx (5 el B per element); mean/rstd
    written and read; W read twice, dW written; b read, db written; per-sample
    vectors (temb twice, emb written and read, scale read, dtemb: 24 K
    elements; d_emb written and read in fp32: 48 KB)."""
    return 5 * el * B * S * D + 16 * B * S + 3 * el * N * D + 2 * el * N + (24576 * el + 49152) * B


def dominant_kernel_bytes(B: int, S: int, el: int = 2) -> int:
    """The backward's main launch: g and x read, dx written (3 el B per
    element), mean/rstd read, the scale half of emb read per sample.  Its
    level-0 token tiles (fp32 pairs, 2 x 24 KB per 32-token tile) are
    implementation overhead, not algorithmic bytes."""
    return 3 * el * B * S * D + 8 * B * S + el * D * B


def residual_algorithmic_bytes(B: int, S: int) -> int:
    """Residual norm site, bf16: the forward reads x and residual and writes h
    and out; the backward reads g_out, g_h, x and h and writes d_residual and
    dx (20 bytes per element in all); mean/rstd written and read (16 per row);
    mod read twice (2 x 18 KB per sample), d_mod written in fp32 (36 KB)."""
    return 20 * B * S * D + 16 * B * S + (2 * 2 * 3 * D + 4 * 3 * D) * B


def residual_dominant_kernel_bytes(B: int, S: int) -> int:
    """The residual backward's main launch: g_out, g_h, x and h read,
    d_residual and dx written (12 bytes per element), mean/rstd read, scale and
    gate read per sample.  Its level-0 tiles are implementation overhead."""
    return 12 * B * S * D + 8 * B * S + 2 * 2 * D * B


def mod6_algorithmic_bytes(B: int) -> int:
    """6-way projection, bf16: W read by the forward and by the backward, dW
    written; bias read, db written; per sample temb read twice, emb and dtemb
    written, d_emb read in fp32."""
    return 3 * 2 * N6 * D + 2 * 2 * N6 + (3 * 2 * D + 2 * N6 + 4 * N6) * B


def mod6_dominant_kernel_bytes(B: int) -> int:
    """The backward's main kernel at B <= 8 (its second launch only finishes
    dtemb): W read, dW and db written, d_emb and temb read."""
    return 2 * 2 * N6 * D + 2 * N6 + (4 * N6 + 2 * D) * B


def proj_out_algorithmic_bytes(T: int) -> int:
    """proj_out, bf16: out read by the forward and by the backward, d_out written
    (6 bytes per element of out); latent written, d_lat read; W read twice, dW
    written; bias read, db written."""
    return 6 * T * D + 4 * T * PO + 6 * PO * D + 4 * PO


def proj_out_dominant_kernel_bytes(T: int) -> int:
    """The backward's main launch (d_out and the dWp partial sums): d_lat, out
    and Wp read, d_out written (the fp32 partials it hands to the chunk sum
    are this design's, not the method's)."""
    return 4 * T * D + 2 * T * PO + 2 * PO * D


def serve_algorithmic_bytes(B: int, S: int) -> int:
    """Serving forward, bf16: x read once, mean and rstd written (fp32), latent
    written; temb, W, bias, Wp, bp read, emb written."""
    T = B * S
    return 2 * T * D + 8 * T + 2 * T * PO + 2 * B * D + 2 * N * D + 2 * N + 2 * B * N + 2 * PO * D + 2 * PO


def serve_dominant_kernel_bytes(B: int, S: int) -> int:
    """The modulate-and-multiply kernel: x, mean, rstd, emb and Wp read; its
    result counted as latent (the fp32 partials it hands to the final add are
    this design's, not the method's)."""
    T = B * S
    return 2 * T * D + 8 * T + 2 * B * N + 2 * PO * D + 2 * T * PO


def pmc_traffic():
    """HBM bytes per launch of the dominant kernel from the committed PMC record,
    or None when the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for src in rec["sources"]:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != rec["sha256"]:
            return None
        return int(rec["fetch_bytes"] + rec["write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="img1024_b1_s4096")
    ap.add_argument("--storage", choices=("bf16", "fp32"), default="bf16",
                    help="tensor storage type (fp32: the fp32-storage entry points)")
    ap.add_argument("--site", choices=("final", "residual", "mod6", "proj_out", "serve"), default="final",
                    help="final: the final modulation (norm_out); residual: a block's residual norm site; "
                         "mod6: a block's 6-way modulation projection; proj_out: the 3072 -> 64 projection; "
                         "serve: the final layer's serving forward (modulation + proj_out, forward only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roles", action="store_true",
                    help="also time the dominant kernel's two roles alone (adaln_norm_mod_bwd_dx and "
                         "adaln_norm_mod_bwd_tiles, each after a flush, 20 launches each; the final site, bf16)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="after the steps, run a plain 512 MiB device copy (PMC byte-counter calibration)")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU's model name with its family / model / stepping numbers
    (a virtualised host may report only a short model name)."""
    info = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (t.strip() for t in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping", "vendor_id") and k not in info:
                    info[k] = v
            elif info:
                break
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    ids = ", ".join(f"{k} {info[k]}" for k in ("vendor_id", "cpu family", "model", "stepping") if k in info)
    return f"{name} ({ids})" if ids else name


def _oracle_fns(site: str):
    from oracle import adaln, modulation, proj_out, residual
    return {"final": (adaln.forward, adaln.backward),
            "residual": (residual.residual_forward, residual.residual_backward),
            "mod6": (modulation.mod6_forward, modulation.mod6_backward),
            "proj_out": (proj_out.proj_out_forward, lambda i, f: proj_out.proj_out_backward(i)),
            "serve": (adaln.forward,
                      lambda i, f: proj_out.proj_out_forward(dict(out=f["out_bits"], W=i["Wp"], bias=i["bp"])))
            }[site]


def _one_thread():
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"


_BARRIER = None


def _init_worker(barrier):
    global _BARRIER
    _BARRIER = barrier
    _one_thread()


def _oracle_worker(args) -> float:
    """One process of the oracle legs: the oracle on its own copy of the
    workload (an independent instance), single-threaded; returns the seconds
    of its forward + backward.  In the all-cores leg every process waits at a
    barrier after drawing its inputs, so the timed passes run side by side."""
    site, workload, seed = args
    inp = _site_inputs(site, workload, seed)
    fwd, bwd = _oracle_fns(site)
    if _BARRIER is not None:
        _BARRIER.wait()
    t0 = time.perf_counter()
    bwd(inp, fwd(inp))
    return time.perf_counter() - t0


def _site_inputs(site: str, workload: str, seed: int = 0) -> dict:
    from synthetic_inputs import (WORKLOADS, make_mod6_inputs, make_proj_out_inputs, make_residual_inputs,
                                  make_workload)
    w = WORKLOADS[workload]
    if site == "residual":
        return make_residual_inputs(w["B"], w["S"], seed=seed)
    if site == "mod6":
        return make_mod6_inputs(w["B"], seed=seed)
    if site == "proj_out":   # a bounded sample: 256 of the workload's tokens
        return make_proj_out_inputs(256, seed=seed)
    inp = make_workload(workload, seed=seed)
    if site == "serve":
        po = make_proj_out_inputs(1, seed=1)
        inp = dict(inp, Wp=po["W"], bp=po["bias"])
    return inp


def _units(site: str, inp: dict):
    if site == "mod6":
        return inp["B"], "samples/s"
    if site == "proj_out":
        return inp["T"], "tokens/s"
    return inp["x"].shape[0] * inp["x"].shape[1], "tokens/s"


def cpu_baseline(site: str, workload: str, reps: int) -> dict:
    """The oracle (NumPy, plain loops, never tuned) timed on this host:
    (i) one thread on the workload batch, `reps` passes (the canonical figure);
    (ii) every available core, each running the oracle single-threaded on an
    independent copy of the workload batch (a process per core), one pass.
    Both legs run in child processes started fresh, none of which touches the
    GPU."""
    import multiprocessing as mp
    cores = len(os.sched_getaffinity(0))
    inp = _site_inputs(site, workload)
    units, unit = _units(site, inp)
    ctx = mp.get_context("spawn")
    with ctx.Pool(1, initializer=_init_worker, initargs=(None,)) as pool:
        dts = pool.map(_oracle_worker, [(site, workload, 0)] * reps, chunksize=reps)
    dt = sum(dts) / len(dts)
    with ctx.Pool(cores, initializer=_init_worker, initargs=(ctx.Barrier(cores),)) as pool:
        wall = max(pool.map(_oracle_worker, [(site, workload, k) for k in range(cores)], chunksize=1))
    what = {"mod6": f"the whole batch (B={inp.get('B')})",
            "proj_out": f"{units} of the workload's tokens",
            "serve": f"the whole workload batch, forward only (final modulation, then proj_out on its bf16 output)"
            }.get(site, f"the whole workload batch ({workload})")
    return {"value": units / dt, "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{what}, fwd+bwd, {reps} passes on one thread, {dt:.2f} s per pass",
            "all_cores": {"value": cores * units / wall, "unit": unit, "cores": cores,
                          "sample": f"{cores} processes, each one pass of the oracle on its own copy of {what} "
                                    f"(seeds 0..{cores - 1}), started together; slowest {wall:.2f} s"},
            "cpu_model": cpu_model(), "host_cores_available": cores}


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, int(q * len(v)))]


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the batch-invariant path has no multi-GPU "
              "mode; --gpus must be 1.", file=sys.stderr)
        return 2

    # the oracle's host timing first, in child processes started before this
    # process touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.site, args.workload,
                           reps=1 if args.site in ("mod6", "proj_out", "serve") else 10)

    import ctypes

    import numpy as np
    import torch

    from invariant_silu_amd import _build, lib
    from synthetic_inputs import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    L = lib.load()
    if not os.path.exists(_build.BENCH_LIB_PATH):
        print(f"{_build.BENCH_LIB_PATH} is missing: run __graft_entry__.build()", file=sys.stderr)
        return 2
    BL = ctypes.CDLL(_build.BENCH_LIB_PATH)
    for fn, argt in (("bench_flush", [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]),
                     ("bench_stream_copy", [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_void_p]),
                     ("bench_event_create", [ctypes.POINTER(ctypes.c_void_p)]),
                     ("bench_event_elapsed", [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]),
                     ("bench_event_destroy", [ctypes.c_void_p])):
        getattr(BL, fn).argtypes = argt
        getattr(BL, fn).restype = ctypes.c_int
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if L.adaln_selftest() != 0:
        print("strict-math self-test failed", file=sys.stderr)
        return 3

    w = WORKLOADS[args.workload]
    B, S = w["B"], w["S"]
    site = args.site
    residual_site, mod6_site, po_site, serve_site = (site == k for k in ("residual", "mod6", "proj_out", "serve"))
    if site != "final" and args.storage != "bf16":
        print(f"--site {site} runs with bf16 storage only", file=sys.stderr)
        return 2
    f32 = args.storage == "fp32"
    el = 4 if f32 else 2
    from synthetic_inputs import (make_mod6_inputs, make_proj_out_inputs, make_residual_inputs,
                                  make_workload)
    if residual_site:
        inp = make_residual_inputs(B, S, seed=0)
        keys = ("x", "residual", "mod", "g_out", "g_h")
    elif mod6_site:
        inp = make_mod6_inputs(B, seed=0)
        keys = ("temb", "W", "bias")
    elif po_site:
        inp = make_proj_out_inputs(B * S, seed=0)
        keys = ("out", "W", "bias", "d_lat")
    else:
        inp = make_workload(args.workload, seed=0, io=args.storage)
        keys = ("x", "temb", "W", "bias", "g")
        if serve_site:
            po = make_proj_out_inputs(1, seed=1)
            inp = dict(inp, Wp=po["W"], bp=po["bias"])
            keys = ("x", "temb", "W", "bias", "Wp", "bp")
    sdt = torch.float32 if f32 else torch.bfloat16

    def to_dev(a):
        if f32:
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = {k: to_dev(inp[k]) for k in keys}
    del inp
    if mod6_site:
        base["d_emb"] = torch.from_numpy(np.ascontiguousarray(make_mod6_inputs(B, seed=0)["d_emb"])).to(dev)
    ws_fw = lib.workspace_bytes(lib.OP_PROJ_FWD, B, 1, D)
    if residual_site:
        ws_bw = lib.workspace_bytes(lib.OP_RESIDUAL_BWD, B, S, D)
    elif mod6_site:
        ws_bw = lib.workspace_bytes(lib.OP_PROJ_BWD, B, 1, D)
    elif po_site:
        ws_fw = lib.workspace_bytes(lib.OP_PROJ_OUT_FWD, B, S, D)
        ws_bw = lib.workspace_bytes(lib.OP_PROJ_OUT_BWD, B, S, D)
    elif serve_site:
        ws_fw = lib.workspace_bytes(lib.OP_FWD_PROJ_OUT, B, S, D)
        ws_bw = 0
    else:
        ws_bw = lib.workspace_bytes(lib.OP_BWD_F32 if f32 else lib.OP_BWD, B, S, D)

    def E(shape, dt=sdt):
        return torch.empty(shape, dtype=dt, device=dev)

    def new_set():
        s = {k: v.clone() for k, v in base.items()}
        s["ws_fw"] = E((max(ws_fw, 256),), torch.uint8)
        s["ws_bw"] = E((max(ws_bw, 256),), torch.uint8)
        if mod6_site:
            s.update(emb=E((B, N6)), dW=E((N6, D)), db=E((N6,)), dtemb=E((B, D)))
        elif serve_site:
            s.update(emb=E((B, N)), latent=E((B, S, PO)), mean=E((B, S), torch.float32),
                     rstd=E((B, S), torch.float32))
        elif po_site:
            s.update(latent=E((B * S, PO)), d_out=E((B * S, D)), dW=E((PO, D)), db=E((PO,)))
        else:
            s.update(out=E((B, S, D)), mean=E((B, S), torch.float32), rstd=E((B, S), torch.float32),
                     dx=E((B, S, D)))
            if residual_site:
                s.update(h=E((B, S, D)), d_residual=E((B, S, D)), d_mod=E((B, 3 * D), torch.float32))
            else:
                s.update(emb=E((B, N)), d_emb=E((B, N), torch.float32), dW=E((N, D)), db=E((N,)),
                         dtemb=E((B, D)))
        return s

    if serve_site:
        step_bytes, k_bytes = serve_algorithmic_bytes(B, S), serve_dominant_kernel_bytes(B, S)
        fwd_name = bwd_name = "adaln_fwd_proj_out"
        k_name = "proj_out_fused_kernel (modulation into LDS, then the fp64 Wp chains)"
    elif po_site:
        step_bytes, k_bytes = proj_out_algorithmic_bytes(B * S), proj_out_dominant_kernel_bytes(B * S)
        fwd_name, bwd_name = "adaln_proj_out_fwd", "adaln_proj_out_bwd"
        k_name = "proj_out_bwd_kernel (d_out = d_lat Wp and the dWp chunk partials in one launch)"
    elif mod6_site:
        if B > 8:
            print("--site mod6 times the B <= 8 backward kernel; use a workload with B <= 8", file=sys.stderr)
            return 2
        step_bytes, k_bytes = mod6_algorithmic_bytes(B), mod6_dominant_kernel_bytes(B)
        fwd_name, bwd_name = "adaln_proj_fwd", "adaln_proj_bwd"
        k_name = f"proj_bwd_small_kernel<{B}, 18432> (dW tiles + da leaf-group blocks)"
    elif residual_site:
        step_bytes, k_bytes = residual_algorithmic_bytes(B, S), residual_dominant_kernel_bytes(B, S)
        fwd_name, bwd_name = "adaln_residual_fwd", "adaln_residual_bwd"
        k_name = "residual_bwd_kernel (dh / dx rows + level-0 tiles of d_shift, d_scale)"
    else:
        step_bytes, k_bytes = algorithmic_bytes(B, S, el), dominant_kernel_bytes(B, S, el)
        fwd_name, bwd_name = ("adaln_fwd_f32", "adaln_bwd_f32") if f32 else ("adaln_fwd", "adaln_bwd")
        k_name = ("norm_mod_bwd_f32_kernel" if f32 else "norm_mod_bwd_kernel<0>") + " (dx rows + level-0 token tiles)"
    kernel_timed = site == "final" and not f32
    if not kernel_timed:
        k_name = f"whole step ({fwd_name})" if serve_site else f"whole step ({fwd_name} + {bwd_name})"
        k_bytes = step_bytes
    # proj_out runs on the fp64 matrix cores and is bound by them, not by HBM:
    # its roofline is fp64 FLOP/s (2 per multiply-add) of the matrix-core work,
    # latent (T x 64 x 3072 multiply-adds) in the forward, d_out and dWp in the
    # backward
    mfma_flops = (2 * B * S * PO * D * (1 if serve_site else 3)) if (po_site or serve_site) else None
    nsets = max(2, math.ceil(3 * MALL_BYTES / step_bytes))
    sets = [new_set() for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    fwd_fn, bwd_fn = getattr(L, fwd_name), getattr(L, bwd_name)

    def fwd(s):
        p = lambda k: s[k].data_ptr()   # noqa: E731
        if serve_site:
            lib.check(fwd_name, fwd_fn(p("temb"), p("W"), p("bias"), p("x"), p("Wp"), p("bp"), p("emb"), p("latent"),
                                       p("mean"), p("rstd"), p("ws_fw"), ws_fw, B, S, D, PO, 1e-6, st))
        elif po_site:
            lib.check(fwd_name, fwd_fn(p("out"), p("W"), p("bias"), p("latent"), p("ws_fw"), ws_fw, B * S, D, PO, st))
        elif mod6_site:
            lib.check(fwd_name, fwd_fn(p("temb"), p("W"), p("bias"), p("emb"), p("ws_fw"), ws_fw, B, D, N6, st))
        elif residual_site:
            lib.check(fwd_name, fwd_fn(p("x"), p("residual"), p("mod"), p("h"), p("out"), p("mean"), p("rstd"),
                                       B, S, D, 1e-6, st))
        else:
            lib.check(fwd_name, fwd_fn(p("temb"), p("W"), p("bias"), p("x"), p("emb"), p("out"), p("mean"),
                                       p("rstd"), B, S, D, 1e-6, st))

    def bwd(s):
        p = lambda k: s[k].data_ptr()   # noqa: E731
        if serve_site:
            return
        if po_site:
            lib.check(bwd_name, bwd_fn(p("d_lat"), p("out"), p("W"), p("d_out"), p("dW"), p("db"), p("ws_bw"), ws_bw,
                                       B * S, D, PO, st))
        elif mod6_site:
            lib.check(bwd_name, bwd_fn(p("d_emb"), p("temb"), p("W"), p("dW"), p("db"), p("dtemb"), p("ws_bw"),
                                       ws_bw, B, D, N6, st))
        elif residual_site:
            lib.check(bwd_name, bwd_fn(p("g_out"), p("g_h"), p("x"), p("h"), p("mean"), p("rstd"), p("mod"),
                                       p("d_residual"), p("dx"), p("d_mod"), p("ws_bw"), ws_bw, B, S, D, st))
        else:
            lib.check(bwd_name, bwd_fn(p("g"), p("x"), p("mean"), p("rstd"), p("emb"), p("temb"), p("W"),
                                       p("dx"), p("d_emb"), p("dW"), p("db"), p("dtemb"), p("ws_bw"),
                                       ws_bw, B, S, D, st))

    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)

    class Events:
        """Timing events of the bench library: recorded by kernel dispatches
        themselves (no event packet of their own in the stream)."""

        def __init__(self, n):
            self.h = []
            for _ in range(n):
                e = ctypes.c_void_p()
                if BL.bench_event_create(ctypes.byref(e)) != 0:
                    raise RuntimeError("bench_event_create failed")
                self.h.append(e.value)

        def ms(self, a, b):
            out = ctypes.c_float()
            if BL.bench_event_elapsed(self.h[a], self.h[b], ctypes.byref(out)) != 0:
                raise RuntimeError("bench_event_elapsed failed")
            return out.value

        def close(self):
            for e in self.h:
                BL.bench_event_destroy(e)

    def flush(ev_start=None, ev_end=None):
        if BL.bench_flush(flush_buf.data_ptr(), FLUSH_BYTES, ev_start, ev_end, st) != 0:
            raise RuntimeError("bench_flush failed")

    # ---- cold caches (the headline): a flush before each phase; a phase runs
    # from the end of the flush before it to the start of the flush after it,
    # both recorded by the flush kernels' own dispatches
    for i in range(args.warmup):
        flush(); fwd(sets[i % nsets]); flush(); bwd(sets[i % nsets])   # noqa: E702
    torch.cuda.synchronize()
    n_cold = max(args.steps, MIN_STAT_STEPS)
    ev = Events(4 * n_cold + 1)   # per step: flush A start, end; flush B start, end; then a closing flush start
    t0 = time.perf_counter()
    for i in range(n_cold):
        s = sets[i % nsets]
        flush(ev.h[4 * i], ev.h[4 * i + 1]); fwd(s)         # noqa: E702
        flush(ev.h[4 * i + 2], ev.h[4 * i + 3]); bwd(s)     # noqa: E702
    flush(ev.h[4 * n_cold], None)
    torch.cuda.synchronize()
    t_cold = time.perf_counter() - t0
    fwd_ms = [ev.ms(4 * i + 1, 4 * i + 2) for i in range(n_cold)]
    bwd_ms = [ev.ms(4 * i + 3, 4 * i + 4) for i in range(n_cold)] if not serve_site else [0.0] * n_cold
    ev.close()
    # the same boundaries with nothing between them: what a phase measured this
    # way costs when it does no work (reported beside the result, not subtracted)
    eev = Events(2 * 20 + 1)
    for i in range(20):
        flush(eev.h[2 * i], eev.h[2 * i + 1])
    flush(eev.h[40], None)
    torch.cuda.synchronize()
    empty_ms = sorted(eev.ms(2 * i + 1, 2 * i + 2) for i in range(20))
    eev.close()
    step_ms = [a + b for a, b in zip(fwd_ms, bwd_ms)]
    timed = step_ms[:args.steps]
    ms_per_step = sum(timed) / len(timed)
    units = B if mod6_site else B * S
    value = units / (ms_per_step / 1e3)

    # ---- the dominant kernel on its own: the backward's first launch (dx and
    # the level-0 token tiles, adaln_norm_mod_bwd_level0), each launch after
    # the same flush as in the step, timed by events its own dispatch records
    n_k = max(MIN_KERNEL_LAUNCHES, args.steps)
    if kernel_timed:
        s0 = sets[0]
        kev = Events(2 * n_k)
        for i in range(n_k):
            flush()
            lib.check("adaln_norm_mod_bwd_level0", L.adaln_norm_mod_bwd_level0(
                s0["g"].data_ptr(), s0["x"].data_ptr(), s0["mean"].data_ptr(), s0["rstd"].data_ptr(),
                s0["emb"].data_ptr(), s0["dx"].data_ptr(), s0["ws_bw"].data_ptr(), ws_bw, B, S, D,
                kev.h[2 * i], kev.h[2 * i + 1], st))
        torch.cuda.synchronize()
        k_ms = sorted(kev.ms(2 * i, 2 * i + 1) for i in range(n_k))
        kev.close()
    else:   # the whole step: fwd + bwd phases
        k_ms = sorted(step_ms)
        n_k = len(k_ms)
    k_mean_ms = sum(k_ms) / len(k_ms)
    if mfma_flops is None:
        achieved, peak, bound, r_unit = k_bytes / (k_mean_ms / 1e3) / 1e9, HBM_PEAK_GBPS, "hbm", "GB/s"
    else:
        achieved, peak, bound, r_unit = mfma_flops / (k_mean_ms / 1e3) / 1e12, FP64_MFMA_PEAK_TFLOPS, "mfma", "TFLOP/s"

    # ---- warm: back-to-back steps over the rotating buffer sets, no flush
    for i in range(args.warmup):
        fwd(sets[i % nsets]); bwd(sets[i % nsets])   # noqa: E702
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        fwd(sets[i % nsets]); bwd(sets[i % nsets])   # noqa: E702
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    # ---- ceiling: the hand-written streaming copy of the step's bytes (half
    # read, half written), after the same flush; and the same copy of four
    # times those bytes, for how the rate grows with size
    def copy_rate(total_bytes):
        cn = (total_bytes // 2 + 255) // 256 * 256
        src = torch.empty(cn, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(cn, dtype=torch.uint8, device=dev)
        cev = Events(2 * 22 + 1)
        for i in range(22):   # timed as the phases are: flush end to next flush start
            flush(cev.h[2 * i], cev.h[2 * i + 1])
            if BL.bench_stream_copy(src.data_ptr(), dst.data_ptr(), cn, None, None, st) != 0:
                raise RuntimeError("bench_stream_copy failed")
        flush(cev.h[44], None)
        torch.cuda.synchronize()
        copy_ms = sorted(cev.ms(2 * i + 1, 2 * i + 2) for i in range(2, 22))
        cev.close()
        del src, dst
        return 2 * cn / (copy_ms[len(copy_ms) // 2] / 1e3) / 1e9

    def kernel_copy_rate(total_bytes):
        """The same copy timed as the dominant kernel is: events recorded by
        its own dispatch, after the same flush; mean of 20."""
        cn = (total_bytes // 2 + 255) // 256 * 256
        src = torch.empty(cn, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(cn, dtype=torch.uint8, device=dev)
        cev = Events(2 * 22)
        for i in range(22):
            flush()
            if BL.bench_stream_copy(src.data_ptr(), dst.data_ptr(), cn, cev.h[2 * i], cev.h[2 * i + 1], st) != 0:
                raise RuntimeError("bench_stream_copy failed")
        torch.cuda.synchronize()
        copy_ms = [cev.ms(2 * i, 2 * i + 1) for i in range(2, 22)]
        cev.close()
        del src, dst
        return 2 * cn / (sum(copy_ms) / len(copy_ms) / 1e3) / 1e9

    copy_gbps = copy_rate(step_bytes)
    copy4_gbps = copy_rate(4 * step_bytes)
    k_copy_gbps = kernel_copy_rate(k_bytes) if (kernel_timed and mfma_flops is None) else None

    roles = None
    if args.roles and kernel_timed:
        # each role of the dominant kernel alone, timed as a phase (flush end to
        # next flush start): the dx rows, then the level-0 tiles
        s0 = sets[0]
        rev = Events(2 * 40 + 1)
        for i in range(40):
            flush(rev.h[2 * i], rev.h[2 * i + 1])
            if i % 2 == 0:
                lib.check("adaln_norm_mod_bwd_dx", L.adaln_norm_mod_bwd_dx(
                    s0["g"].data_ptr(), s0["x"].data_ptr(), s0["mean"].data_ptr(), s0["rstd"].data_ptr(),
                    s0["emb"].data_ptr(), s0["dx"].data_ptr(), B, S, D, st))
            else:
                lib.check("adaln_norm_mod_bwd_tiles", L.adaln_norm_mod_bwd_tiles(
                    s0["g"].data_ptr(), s0["x"].data_ptr(), s0["mean"].data_ptr(), s0["rstd"].data_ptr(),
                    s0["ws_bw"].data_ptr(), ws_bw, B, S, D, st))
        flush(rev.h[80], None)
        torch.cuda.synchronize()
        ph = [rev.ms(2 * i + 1, 2 * i + 2) for i in range(40)]
        rev.close()
        roles = {"dx_rows_phase_ms": round(_pct(ph[0::2], 0.5), 5), "tiles_phase_ms": round(_pct(ph[1::2], 0.5), 5),
                 "note": "each role alone after the same flush, timed as a phase, medians of 20"}

    if args.copy_calib:
        n = 512 << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    gbps = lambda ms: step_bytes / (ms / 1e3) / 1e9   # noqa: E731
    result = {
        "metric": {"final": METRIC, "residual": METRIC_RESIDUAL, "mod6": METRIC_MOD6,
                   "proj_out": METRIC_PROJ_OUT, "serve": METRIC_SERVE}[site],
        "value": round(value, 1),
        "unit": "samples/s" if mod6_site else "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "S": None if mod6_site else S, "D": D,
                   "N": {"mod6": N6, "proj_out": PO}.get(site, N), "site": site,
                   "storage": args.storage,
                   "accumulate": "fp64",
                   "outlier_rows": w["outlier_frac"] if site in ("final", "serve") else 0.0,
                   "timing": ("cold caches: before each phase a flush writes and reads back "
                              f"{FLUSH_BYTES >> 20} MiB; a phase runs from the end of the flush before it to the "
                              "start of the flush after it (HIP events recorded by the flush kernels' own "
                              "dispatches, so launch gaps inside the phase count and no event packet does); "
                              "ms_per_step = mean over the timed steps of (forward + backward)"),
                   "step_algorithmic_bytes": step_bytes,
                   "step_gbps": round(gbps(ms_per_step), 1),
                   "step_frac_of_peak": round(gbps(ms_per_step) / HBM_PEAK_GBPS, 4),
                   "cold_steps_measured": n_cold,
                   "cold_median_ms": round(_pct(step_ms, 0.5), 5),
                   "cold_p10_ms": round(_pct(step_ms, 0.1), 5),
                   "cold_p90_ms": round(_pct(step_ms, 0.9), 5),
                   "cold_fwd_median_ms": round(_pct(fwd_ms, 0.5), 5),
                   "cold_bwd_median_ms": round(_pct(bwd_ms, 0.5), 5),
                   "cold_wall_s_incl_flushes": round(t_cold, 3),
                   "empty_phase_ms": round(empty_ms[len(empty_ms) // 2], 5),
                   **({"roles": roles} if roles else {}),
                   "warm_ms_per_step": round(warm_ms, 5),
                   "warm_tokens_per_s": round(units / (warm_ms / 1e3), 1),
                   "warm_step_gbps": round(gbps(warm_ms), 1),
                   "warm_note": ("back-to-back steps over buffer sets rotated so that no step finds the previous "
                                 "step's data in the 256 MB memory-side cache; inside a step the backward finds "
                                 "x and W that the forward read there"),
                   "buffer_sets": nsets,
                   "copy_ceiling_gbps": round(copy_gbps, 1),
                   "copy_ceiling_kernel": ("bench_stream_copy: hand-written, 16 B per lane, after the same flush, "
                                           "timed as a phase, median of 20"),
                   "copy_4x_step_bytes_gbps": round(copy4_gbps, 1),
                   "step_frac_of_copy_ceiling": round(gbps(ms_per_step) / copy_gbps, 4)},
        "roofline": {"bound": bound,
                     "kernel": k_name,
                     "achieved": round(achieved, 1 if mfma_flops is None else 2), "peak": peak, "unit": r_unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": None if (f32 or site != "final") else pmc_traffic(),
                     **({"bytes_per_launch": k_bytes} if mfma_flops is None else
                        {"fp64_flops_per_step": mfma_flops, "step_bytes": k_bytes}),
                     "avg_launch_ms": round(k_mean_ms, 5),
                     **({"copy_same_bytes_gbps": round(k_copy_gbps, 1),
                         "frac_of_copy_same_bytes": round(achieved / k_copy_gbps, 4),
                         "copy_note": ("bench_stream_copy of the kernel's algorithmic bytes (half read, half "
                                       "written) after the same flush, timed by its own dispatch events")}
                        if k_copy_gbps else {}),
                     "timed_launches": n_k,
                     "timing": ("HIP events recorded by the dispatch of adaln_norm_mod_bwd_level0 (this kernel "
                                "alone) on the step's stream, each launch after the same flush as in the step"
                                if kernel_timed else
                                "the step's forward + backward phase events (this site has no single dominant "
                                "kernel timed on its own)"),
                     "median_launch_ms": round(_pct(k_ms, 0.5), 5),
                     "p10_launch_ms": round(_pct(k_ms, 0.1), 5),
                     "p90_launch_ms": round(_pct(k_ms, 0.9), 5)},
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
