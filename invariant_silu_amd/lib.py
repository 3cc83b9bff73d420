"""ctypes binding of ``libadaln.so`` (declared in include/adaln.h).

Argument marshalling only: every step of the operator runs in the library's
HIP kernels.  Loading fails loudly when the library has not been built; there
is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libadaln.so")

OK = 0
ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_DEVICE, ERR_WORKSPACE, ERR_OVERLAP, ERR_LAUNCH, ERR_SCRATCH = range(-1, -9, -1)
(OP_PROJ_FWD, OP_NORM_MOD_BWD, OP_PROJ_BWD, OP_TOKEN_TREE_SUM, OP_BWD, OP_BWD_F32, OP_RESIDUAL_BWD,
 OP_PROJ_OUT_BWD, OP_PROJ_OUT_FWD, OP_FWD_PROJ_OUT) = range(1, 11)

EXPORTS = ("adaln_fwd", "adaln_bwd", "adaln_fwd_f32", "adaln_bwd_f32", "adaln_residual_fwd", "adaln_residual_bwd",
           "adaln_site_fwd", "adaln_site_bwd",
           "adaln_proj_out_fwd", "adaln_proj_out_bwd", "adaln_fwd_proj_out", "adaln_proj_fwd", "adaln_norm_mod_fwd", "adaln_norm_mod_bwd", "adaln_proj_bwd",
           "adaln_proj_bwd_acc",
           "token_tree_sum", "adaln_norm_mod_bwd_dx", "adaln_norm_mod_bwd_tiles", "token_tree_fold",
           "adaln_norm_mod_bwd_noalloc",
           "adaln_norm_mod_bwd_level0", "adaln_workspace_bytes", "adaln_selftest", "adaln_strerror",
           "adaln_abi_version")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SIGS = {
    "adaln_proj_fwd": ([_P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_fwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_float, _P], ctypes.c_int),
    "adaln_bwd": ([_P] * 13 + [_SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_residual_fwd": ([_P] * 7 + [_I64, _I64, _I64, ctypes.c_float, _P], ctypes.c_int),
    "adaln_residual_bwd": ([_P] * 11 + [_SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_proj_out_fwd": ([_P] * 5 + [_SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_site_fwd": ([_P] * 5 + [_I64] + [_P] * 4 + [_I64, _I64, _I64, ctypes.c_float, _P], ctypes.c_int),
    "adaln_site_bwd": ([_P] * 8 + [_I64] + [_P] * 5 + [_I64, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_proj_out_bwd": ([_P] * 7 + [_SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_fwd_proj_out": ([_P] * 11 + [_SZ, _I64, _I64, _I64, _I64, ctypes.c_float, _P], ctypes.c_int),
    "adaln_fwd_f32": ([_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_float, _P], ctypes.c_int),
    "adaln_bwd_f32": ([_P] * 13 + [_SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_norm_mod_fwd": ([_P, _P, _P, _P, _P, _I64, _I64, _I64, ctypes.c_float, _P], ctypes.c_int),
    "adaln_norm_mod_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_proj_bwd": ([_P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_proj_bwd_acc": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "token_tree_sum": ([_P, _P, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_norm_mod_bwd_dx": ([_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_norm_mod_bwd_tiles": ([_P, _P, _P, _P, _P, _SZ, _I64, _I64, _I64, _P], ctypes.c_int),
    "token_tree_fold": ([_P, _SZ, _P, _I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_norm_mod_bwd_noalloc": ([_P] * 7 + [_I64, _I64, _I64, _P], ctypes.c_int),
    "adaln_workspace_bytes": ([ctypes.c_int, _I64, _I64, _I64], _SZ),
    "adaln_selftest": ([], ctypes.c_int),
    "adaln_norm_mod_bwd_level0": ([_P] * 7 + [_SZ, _I64, _I64, _I64, _P, _P, _P], ctypes.c_int),
    "adaln_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "adaln_abi_version": ([], ctypes.c_int),
}

# ADALN_ABI_VERSION of include/adaln.h that the signatures above describe
ABI_VERSION = 17

_lock = threading.Lock()
_lib = None


class AdaLNError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        try:
            # load PyTorch's HIP runtime first so the library binds to the same one
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with __graft_entry__.build() "
                              "(or python -m invariant_silu_amd._build); there is no fallback")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        found = lib.adaln_abi_version()
        if found != ABI_VERSION:
            raise ImportError(f"{path} has ABI version {found}, this binding expects {ABI_VERSION}: "
                              "rebuild it with __graft_entry__.build()")
        _lib = lib
        return lib


def strerror(status: int) -> str:
    return load().adaln_strerror(status).decode()


def check(fn: str, status: int) -> None:
    if status != OK:
        raise AdaLNError(fn, status, strerror(status))


def call(fn: str, *args) -> None:
    """Call an entry point and raise AdaLNError on a non-zero status."""
    check(fn, getattr(load(), fn)(*args))


def workspace_bytes(op: int, B: int, S: int, H: int) -> int:
    return int(load().adaln_workspace_bytes(op, B, S, H))
