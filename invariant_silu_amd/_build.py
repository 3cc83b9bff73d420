"""Build the HIP library ``libadaln.so`` in-tree with hipcc for gfx950.

Flags: -O3, -ffp-contract=off (no implicit fused multiply-add: every float
operation in the kernels is one IEEE operation), correctly rounded fp32
division and square root, fp32 denormals kept (HIP's default for gfx950),
packed fp32 vector instructions disabled on the device pass, matrix-core
accumulators in VGPRs, code object v5.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB_NAME = "libadaln.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

# measurement helpers for bench.py (cache flush, streaming copy): a library of
# their own, not part of the operator's
BENCH_SOURCE = "bench_util.hip"
BENCH_LIB_PATH = os.path.join(PKG, "libadaln_bench.so")

SOURCES = ["api.cpp", "fwd.hip", "norm_bwd.hip", "site.hip", "proj_bwd.hip", "proj_out.hip", "token_tree.hip",
           "fp32.hip", "selftest.hip", "noalloc.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: a runtime loop over an MFMA
    # chain otherwise copies every accumulator between VGPRs and AGPRs on
    # each iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err)


def build(verbose: bool = True) -> str:
    """Compile every source and link ``libadaln.so``; returns its path."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    bench_obj = os.path.join(objdir, os.path.splitext(BENCH_SOURCE)[0] + ".o")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        list(ex.map(_compile, SOURCES + [BENCH_SOURCE], objs + [bench_obj]))
    for out, ins in ((LIB_PATH, objs), (BENCH_LIB_PATH, [bench_obj])):
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-fno-gpu-rdc", *ins, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
        os.replace(tmp, out)
        if verbose:
            print(f"built {out}")
    return LIB_PATH


if __name__ == "__main__":
    build()
