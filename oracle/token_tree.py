"""CPU models of the fixed token-sum trees (test infrastructure only).

RL-Kernel pull request 538 reduces d_scale / d_shift over the S tokens of each
sample with a tree whose shape depends only on S, never on the batch size or
the sample's position in the batch ("What": fixed 32-way balanced trees applied
recursively until one value remains).  Its review thread records two versions:

* ``plain_tree_sum`` -- the first version: each group of 32 values is added as
  a balanced pairwise tree, recursively.  The review reports it returns 6020 on
  the cancellation case (S = 6032, one token +2^26 and one -2^26 among ones),
  where the exact sum is 6030.  Kept as the "has teeth" control.
* ``tree_sum`` -- the fix: every 32-token tile is summed in ascending token
  order with Neumaier compensation; the tile sums and their corrections are
  folded level by level (32 children per node, ascending); a single IEEE add
  of sum and correction gives the result.  The H100 results section reports
  6030 on the cancellation case.

Reading of the fold (the pages do not spell it out): a
node visits its children in ascending order; for each child it takes one
Neumaier step on the child's sum (s, c updated) and then adds the child's
correction into c.  Tiles restart at token 0 of every sample.  Accumulators
start at +0.  With one tile (S <= 32) the result is the tile's s + c.

Pinned by tests/test_oracle_pins.py: 6030 for every placement of the two large
tokens (the pages' worked example, tests/golden/cancellation_probe.json), the
plain tree's 6020, exact results within a few ulp of ``math.fsum`` on random
data, and byte-neutrality to trailing zero tokens.
"""

from __future__ import annotations

import math

import numpy as np

TILE = 32


def _neumaier_step(s, c, x):
    t = s + x
    big = np.abs(s) >= np.abs(x)
    e = np.where(big, (s - t) + x, (x - t) + s)
    return t, c + e


def _level0(x):
    """x: float32 [B, S, H] -> tile sums and corrections [B, T0, H]."""
    B, S, H = x.shape
    T0 = math.ceil(S / TILE)
    s = np.zeros((B, T0, H), np.float32)
    c = np.zeros((B, T0, H), np.float32)
    for p in range(TILE):
        idx = np.arange(T0) * TILE + p
        valid = idx < S
        if not valid.any():
            break
        xv = np.zeros((B, T0, H), np.float32)
        xv[:, valid, :] = x[:, idx[valid], :]
        t, cn = _neumaier_step(s, c, xv)
        s = np.where(valid[None, :, None], t, s)
        c = np.where(valid[None, :, None], cn, c)
    return s, c


def _fold(vs, vc):
    """One level: groups of 32 consecutive nodes -> one node each."""
    B, T, H = vs.shape
    Tn = math.ceil(T / TILE)
    s = np.zeros((B, Tn, H), np.float32)
    c = np.zeros((B, Tn, H), np.float32)
    for p in range(TILE):
        idx = np.arange(Tn) * TILE + p
        valid = idx < T
        if not valid.any():
            break
        xs = np.zeros((B, Tn, H), np.float32)
        xc = np.zeros((B, Tn, H), np.float32)
        xs[:, valid, :] = vs[:, idx[valid], :]
        xc[:, valid, :] = vc[:, idx[valid], :]
        t, cn = _neumaier_step(s, c, xs)
        cn = cn + xc
        s = np.where(valid[None, :, None], t, s)
        c = np.where(valid[None, :, None], cn, c)
    return s, c


def tree_sum(x) -> np.ndarray:
    """Compensated 32-token tree sum over axis 1 of a float32 [B, S, H] array."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 3 or x.shape[1] < 1:
        raise ValueError("expected [B, S, H] with S >= 1")
    s, c = _level0(x)
    while s.shape[1] > 1:
        s, c = _fold(s, c)
    return (s[:, 0, :] + c[:, 0, :]).astype(np.float32)


def tree_levels(S: int) -> list:
    """Node counts per level: [T0, T1, ..., 1]."""
    out = [math.ceil(S / TILE)]
    while out[-1] > 1:
        out.append(math.ceil(out[-1] / TILE))
    return out


def _pairwise32(v):
    """Balanced pairwise sum of up to 32 values along axis 1 (zero-padded to 32)."""
    B, n, H = v.shape
    buf = np.zeros((B, TILE, H), np.float32)
    buf[:, :n, :] = v
    while buf.shape[1] > 1:
        buf = (buf[:, 0::2, :] + buf[:, 1::2, :]).astype(np.float32)
    return buf[:, 0, :]


def plain_tree_sum(x) -> np.ndarray:
    """The uncompensated tree: balanced pairwise sums of 32-groups, recursively."""
    v = np.asarray(x, dtype=np.float32)
    while True:
        B, T, H = v.shape
        groups = [_pairwise32(v[:, i:i + TILE, :]) for i in range(0, T, TILE)]
        v = np.stack(groups, axis=1)
        if v.shape[1] == 1:
            return v[:, 0, :]
