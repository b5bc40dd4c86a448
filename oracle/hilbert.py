"""Hilbert-curve token order, oracle side (integer NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests and the bench's CPU leg, never by the product
path; shares no code with the HIP kernels.

Source: the DFSAttn page (abstract): tokens are reordered along a Hilbert curve so that blocks
of consecutive tokens are compact regions of the video.  The page gives no construction.
Reading used here: the 3D Hilbert curve of the smallest cube of side 2^b holding the T x H x W
grid, axes (t, h, w), in J. Skilling's formulation ("Programming the Hilbert curve", AIP Conf.
Proc. 707, 2004): the axis coordinates are turned into the curve's "transposed" index by
undoing the excess work of each level (inverting or exchanging low bits per axis), a Gray code
across the axes and a final correction; the index is then the bits of the transposed form
interleaved from the most significant level down.  Tokens of the grid are ordered by that
index (cells of the cube outside the grid are skipped); blocks are B consecutive tokens of
that order, padded at the end exactly as for the 3D-tile order.
"""
from __future__ import annotations

import numpy as np


def cube_bits(T: int, H: int, W: int) -> int:
    b = 1
    while (1 << b) < max(T, H, W):
        b += 1
    return b


def hilbert_index(t, h, w, bits: int) -> np.ndarray:
    """Hilbert index (0 .. 8^bits - 1) of cells (t, h, w) of the 2^bits cube."""
    X = [np.asarray(t, np.int64).copy(), np.asarray(h, np.int64).copy(),
         np.asarray(w, np.int64).copy()]
    n = 3
    M = 1 << (bits - 1)
    Q = M
    while Q > 1:                      # undo excess work, level by level
        P = Q - 1
        for i in range(n):
            hit = (X[i] & Q) != 0
            inv = X[0] ^ P                                # invert the low bits of axis 0
            tt = (X[0] ^ X[i]) & P                        # or exchange them with axis i
            x0_ex = X[0] ^ tt
            xi_ex = X[i] ^ tt
            X0_new = np.where(hit, inv, x0_ex)
            Xi_new = np.where(hit, X[i], xi_ex)
            if i == 0:
                X[0] = np.where(hit, inv, X[0])           # exchange of axis 0 with itself: no-op
            else:
                X[0], X[i] = X0_new, Xi_new
        Q >>= 1
    for i in range(1, n):             # Gray encode
        X[i] = X[i] ^ X[i - 1]
    tcor = np.zeros_like(X[0])
    Q = M
    while Q > 1:
        tcor = np.where((X[n - 1] & Q) != 0, tcor ^ (Q - 1), tcor)
        Q >>= 1
    for i in range(n):
        X[i] = X[i] ^ tcor
    idx = np.zeros_like(X[0])
    for bit in range(bits - 1, -1, -1):                   # interleave, top level first
        for i in range(n):
            idx = (idx << 1) | ((X[i] >> bit) & 1)
    return idx


def hilbert_perm(T: int, H: int, W: int) -> np.ndarray:
    """pi[n] = Hilbert-order position of raster token n = (t*H + h)*W + w."""
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    key = hilbert_index(t.ravel(), h.ravel(), w.ravel(), cube_bits(T, H, W))
    order = np.argsort(key, kind="stable")                # order[pos] = raster token
    pi = np.empty_like(order)
    pi[order] = np.arange(order.size)
    return pi.astype(np.int64)


def hilbert_order(T: int, H: int, W: int) -> np.ndarray:
    """order[pos] = raster token at position pos (the table the GPU path takes)."""
    pi = hilbert_perm(T, H, W)
    order = np.empty_like(pi)
    order[pi] = np.arange(pi.size)
    return order
