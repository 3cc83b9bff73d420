"""Batch-invariant AdaLN final modulation (Qwen-Image ``norm_out``) for MI355X.

The operator lives in the HIP library ``libadaln.so`` (C ABI in
``include/adaln.h``); ``lib`` binds it with ctypes and ``ops`` wraps it for
PyTorch tensors (device memory and streams only).
"""

from . import lib  # noqa: F401

__all__ = ["lib"]
