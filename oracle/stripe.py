"""Static periodic-stripe block masks, oracle side (fp64/int NumPy).

TEST INFRASTRUCTURE ONLY: imported by the tests and the bench's CPU leg, never by the product
path; shares no code with the HIP kernels.

Source: the PSA page ("Parameterized Stripe Attention for Efficient Video Generation",
"Approach"): the attention of video DiTs concentrates on bands that repeat along the
diagonal, which one mask of six parameters M(Tw, To, Ts, Sw, So, Ss) per head covers, executed
by a single block-sparse kernel.  The
page names the parameters but does not define them.  Reading used here (T = temporal,
S = spatial; w = stripe width, o = offset, s = period), on the block grid of the 3D-tile
order:

* a block's grid coordinates are those of the tile that holds its first token: temporal tile
  index bt = t // tt and spatial tile index bs = (h // th) * nW + (w // tw), nW = ceil(W / tw);
* query block i keeps key block j iff
      (bt_j - bt_i - To) mod Ts < Tw   and   (bs_j - bs_i - So) mod Ss < Sw,
  with mod the non-negative remainder, 1 <= Tw <= Ts and 1 <= Sw <= Ss;
* the columns of a row are listed ascending (CSR), one parameter set per head.
"""
from __future__ import annotations

import numpy as np

from .bsa_oracle import num_blocks, tile_perm


def check_params(p):
    Tw, To, Ts, Sw, So, Ss = (int(x) for x in p)
    if not (1 <= Tw <= Ts and 1 <= Sw <= Ss):
        raise ValueError(f"stripe parameters need 1 <= Tw <= Ts and 1 <= Sw <= Ss, got {p}")
    return Tw, To, Ts, Sw, So, Ss


def block_coords(T: int, H: int, W: int, tile, B: int, pi=None):
    """(bt, bs) of every block: the tile coordinates of the block's first token (blocks of the
    3D-tile order, or of the token order pi[n] = position of raster token n)."""
    tt, th, tw = tile
    N = T * H * W
    pi = tile_perm(T, H, W, tile) if pi is None else np.asarray(pi)
    order = np.argsort(pi)                              # order[pos] = raster token at pos
    first = order[np.arange(num_blocks(N, B)) * B]
    t, h, w = first // (H * W), (first // W) % H, first % W
    nW = -(-W // tw)
    return (t // tt).astype(np.int64), ((h // th) * nW + w // tw).astype(np.int64)


def stripe_keep(bt, bs, p) -> np.ndarray:
    """Dense [n, n] bool mask of one head."""
    Tw, To, Ts, Sw, So, Ss = check_params(p)
    dt = bt[None, :] - bt[:, None] - To
    ds = bs[None, :] - bs[:, None] - So
    return (np.mod(dt, Ts) < Tw) & (np.mod(ds, Ss) < Sw)


def stripe_mask(T: int, H: int, W: int, tile, B: int, params, batch: int = 1, pi=None):
    """CSR (row_ptr, col_idx) over rows (b, h, i) for params[h] = (Tw, To, Ts, Sw, So, Ss)."""
    bt, bs = block_coords(T, H, W, tile, B, pi)
    counts, cols = [], []
    for _ in range(batch):
        for p in params:
            keep = stripe_keep(bt, bs, p)
            for i in range(keep.shape[0]):
                c = np.nonzero(keep[i])[0]
                counts.append(c.size)
                cols.append(c)
    row_ptr = np.zeros(len(counts) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols).astype(np.int64) if cols else np.zeros(0, np.int64)
    return row_ptr, col_idx
