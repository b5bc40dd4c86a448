"""CPU oracle for training-free block-sparse video attention (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links this module:
only the tests, the package's smoke check and the bench's CPU-baseline leg use it.  It shares
no code with the HIP path.

What is computed, and where the pages define it:

* FVAttn (page "FVAttn: Adaptive Sparse Attention with Runtime Load Balancing for Video
  Generation", abstract): a routing frontend made of video-aware block organization, Top-p
  routing and a Top-k safety floor produces a materialized block mask; sparse attention then
  runs over that mask.  The pages give no formula for any step; the plain readings used here
  are listed beside each function:
  - video-aware block organization = tokens of the T x H x W latent grid regrouped into 3D
    tiles (tiles in lexicographic order, row-major inside a tile, edge tiles truncated), then
    cut into blocks of B consecutive tokens;
  - block scores = scaled dot products of per-block mean-pooled queries and keys;
  - Top-p = the smallest prefix, in descending score order, whose block-level softmax mass
    reaches p; Top-k floor = at least k blocks.
* Exact block-sparse attention with an online softmax: the pages describe block-sparse
  kernels (PSA page, "Approach": one block-sparse kernel; DFSAttn abstract: block sparse
  attention; VC-Attention abstract: the row sum an online softmax keeps).  The online softmax
  is an evaluation order of the exact softmax over the selected keys, so the oracle is that
  definition written out: logsumexp with the maximum shifted out, then weights times V.

Everything here is fp64.  bf16 inputs arrive as uint16 bit patterns and are widened exactly.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
from threadpoolctl import threadpool_limits


# ---------------------------------------------------------------------------------------
# encodings
# ---------------------------------------------------------------------------------------
def widen_bf16(u) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.asarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------
# video-aware block organization (FVAttn abstract; 3D tiles, edge tiles truncated)
# ---------------------------------------------------------------------------------------
def num_blocks(N: int, B: int) -> int:
    return -(-N // B)


def padded_len(N: int, B: int) -> int:
    return num_blocks(N, B) * B


def tile_perm(T: int, H: int, W: int, tile) -> np.ndarray:
    """pi[n] = tile-order position of raster token n = (t*H + h)*W + w.

    Tiles are visited in (it, ih, iw) order, the last tile along an axis is truncated to what
    is left of the grid, and tokens inside a tile are row-major (t, h, w).  Position of token
    (t, h, w): all complete tile-slabs before it (it*tt*H*W tokens), then the tile rows of its
    slab before it (et*ih*th*W), then the tiles of its tile row before it (et*eh*iw*tw), then
    its row-major offset inside its own et x eh x ew tile."""
    tt, th, tw = tile
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    it, ih, iw = t // tt, h // th, w // tw
    rt, rh, rw = t % tt, h % th, w % tw
    et = np.minimum(tt, T - it * tt)
    eh = np.minimum(th, H - ih * th)
    ew = np.minimum(tw, W - iw * tw)
    pos = (it * tt * H * W + et * ih * th * W + et * eh * iw * tw
           + (rt * eh + rh) * ew + rw)
    return pos.astype(np.int64)


def tile_perm_by_sort(T: int, H: int, W: int, tile) -> np.ndarray:
    """Second formulation of the same permutation: sort raster tokens by the key
    (it, ih, iw, rt, rh, rw) and read off each token's rank."""
    tt, th, tw = tile
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    keys = (w % tw, h % th, t % tt, w // tw, h // th, t // tt)   # lexsort: last key primary
    order = np.lexsort(keys)              # order[pos] = raster index at tile position pos
    pi = np.empty_like(order)
    pi[order] = np.arange(order.size)
    return pi.astype(np.int64)


def reorder(x, T: int, H: int, W: int, tile, B: int, pi=None) -> np.ndarray:
    """[batch, N, heads, D] raster -> [batch, heads, Npad, D] tile order (or the token order
    pi[n] = position of raster token n, e.g. the Hilbert order); pad rows are 0."""
    x = np.asarray(x)
    b, N, h, D = x.shape
    assert N == T * H * W
    pi = tile_perm(T, H, W, tile) if pi is None else np.asarray(pi)
    out = np.zeros((b, h, padded_len(N, B), D), dtype=x.dtype)
    out[:, :, pi, :] = np.transpose(x, (0, 2, 1, 3))
    return out


def inverse_reorder(xt, T: int, H: int, W: int, tile, pi=None) -> np.ndarray:
    """[batch, heads, Npad, D] tile (or pi) order -> [batch, N, heads, D] raster; pad rows
    dropped."""
    xt = np.asarray(xt)
    N = T * H * W
    pi = tile_perm(T, H, W, tile) if pi is None else np.asarray(pi)
    return np.ascontiguousarray(np.transpose(xt[:, :, pi, :], (0, 2, 1, 3)))


# ---------------------------------------------------------------------------------------
# block scoring (mean-pooled Q and K per block, scaled dot product, block softmax)
# ---------------------------------------------------------------------------------------
def block_ranges(N: int, B: int):
    """Real token positions [lo, hi) of each block; only the last block can be short."""
    n = num_blocks(N, B)
    return [(j * B, min((j + 1) * B, N)) for j in range(n)]


def pool(xt, N: int, B: int) -> np.ndarray:
    """Per-block mean over the block's real tokens: [b, h, Npad, D] -> [b, h, n_blk, D]."""
    xt = np.asarray(xt, dtype=np.float64)
    out = np.empty(xt.shape[:2] + (num_blocks(N, B), xt.shape[3]), dtype=np.float64)
    for j, (lo, hi) in enumerate(block_ranges(N, B)):
        out[:, :, j, :] = xt[:, :, lo:hi, :].sum(axis=2) / (hi - lo)
    return out


def block_scores(qbar, kbar, scale: float) -> np.ndarray:
    """s[..., i, j] = scale * <qbar_i, kbar_j>."""
    return scale * np.matmul(qbar, np.swapaxes(kbar, -1, -2))


def block_mass(s) -> np.ndarray:
    """Softmax of the scores over the key-block axis (max shifted out)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------------------
# Top-p routing with a Top-k floor (FVAttn abstract)
# ---------------------------------------------------------------------------------------
@dataclass
class RowRoute:
    order: np.ndarray      # key blocks by score descending, ties -> smaller index first
    cum: np.ndarray        # cumulative block mass along `order`
    k_p: int               # Top-p count
    count: int             # final count max(k_p, k_floor), capped at n_blk
    cols: np.ndarray       # selected key blocks, ascending


def route_row(s_row, top_p: float, k_floor: int, mass_row=None) -> RowRoute:
    """Route one query block.

    Order the key blocks by score (descending; equal scores keep the smaller block index
    first), accumulate their block mass along that order, keep the shortest prefix whose mass
    reaches top_p (p >= 1 keeps every block; p <= 0 keeps none; if rounding keeps the total
    below p, keep every block), then raise the count to the floor and cap it at n_blk."""
    s_row = np.asarray(s_row, dtype=np.float64)
    n = s_row.size
    P = block_mass(s_row) if mass_row is None else np.asarray(mass_row, dtype=np.float64)
    order = np.lexsort((np.arange(n), -s_row))
    cum = np.cumsum(P[order])
    if top_p >= 1.0:
        k_p = n
    elif top_p <= 0.0:
        k_p = 0
    else:
        hit = np.nonzero(cum >= top_p)[0]
        k_p = int(hit[0]) + 1 if hit.size else n
    c = min(n, max(k_p, int(k_floor)))
    cols = np.sort(order[:c])
    return RowRoute(order=order, cum=cum, k_p=k_p, count=c, cols=cols)


@dataclass
class Routing:
    row_ptr: np.ndarray            # [rows + 1] int64
    col_idx: np.ndarray            # [nnz] int64, ascending within a row
    scores: np.ndarray             # [b, h, n_blk, n_blk] fp64
    mass: np.ndarray               # [b, h, n_blk, n_blk] fp64
    rows: List[RowRoute]           # rows in (batch, head, q-block) order

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])


def route(qt, kt, N: int, B: int, top_p: float, k_floor: int, scale: float) -> Routing:
    """Full routing frontend on tile-ordered Q, K ([b, h, Npad, D], fp64 or bf16 bits)."""
    qt = widen_bf16(qt) if np.asarray(qt).dtype == np.uint16 else np.asarray(qt, np.float64)
    kt = widen_bf16(kt) if np.asarray(kt).dtype == np.uint16 else np.asarray(kt, np.float64)
    qbar, kbar = pool(qt, N, B), pool(kt, N, B)
    s = block_scores(qbar, kbar, scale)
    P = block_mass(s)
    b, h, n, _ = s.shape
    rows, counts, cols = [], [], []
    for bi in range(b):
        for hi in range(h):
            for i in range(n):
                r = route_row(s[bi, hi, i], top_p, k_floor, P[bi, hi, i])
                rows.append(r)
                counts.append(r.count)
                cols.append(r.cols)
    row_ptr = np.zeros(len(rows) + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.concatenate(cols).astype(np.int64) if cols else np.zeros(0, np.int64)
    return Routing(row_ptr=row_ptr, col_idx=col_idx, scores=s, mass=P, rows=rows)


# ---------------------------------------------------------------------------------------
# exact attention over the selected key blocks
# ---------------------------------------------------------------------------------------
def _attend(q, k, v, scale):
    """Exact softmax attention of query rows q over keys k/values v: (O, LSE)."""
    logits = scale * (q @ k.T)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    l = e.sum(axis=1, keepdims=True)
    return (e @ v) / l, (m + np.log(l))[:, 0]


def sparse_attn(qt, kt, vt, row_ptr, col_idx, N: int, B: int, scale: float,
                heads: Optional[Sequence[int]] = None, qblocks=None, threads: int = 0):
    """Block-gather formulation: for each (batch, head, q-block) row, one product against the
    concatenated real tokens of the row's selected key blocks (ascending block order).

    Inputs [b, h, Npad, D] (fp64 or bf16 bits); CSR rows in (batch, head, q-block) order.
    Returns O [b, h, Npad, D] fp64 and LSE [b, h, Npad] fp64; rows that were not computed
    (pad queries, or rows outside `heads`/`qblocks`) hold NaN."""
    def f64(x):
        x = np.asarray(x)
        return widen_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64, copy=False)
    qt, kt, vt = f64(qt), f64(kt), f64(vt)
    b, h, Npad, D = qt.shape
    n = num_blocks(N, B)
    rng = block_ranges(N, B)
    O = np.full((b, h, Npad, D), np.nan)
    LSE = np.full((b, h, Npad), np.nan)
    heads = range(h) if heads is None else heads
    qblocks = range(n) if qblocks is None else qblocks

    def one(bh):
        bi, hi = bh
        for i in qblocks:
            r = (bi * h + hi) * n + i
            sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
            keys = np.concatenate([np.arange(*rng[j]) for j in sel])
            lo, hi_ = rng[i]
            o, lse = _attend(qt[bi, hi, lo:hi_], kt[bi, hi, keys], vt[bi, hi, keys], scale)
            O[bi, hi, lo:hi_] = o
            LSE[bi, hi, lo:hi_] = lse

    jobs = [(bi, hi) for bi in range(b) for hi in heads]
    nthr = threads or min(os.cpu_count() or 1, len(jobs))
    if nthr > 1:
        # heads run in parallel; one BLAS thread each avoids oversubscription
        with threadpool_limits(1), ThreadPoolExecutor(nthr) as ex:
            list(ex.map(one, jobs))
    else:
        for j in jobs:
            one(j)
    return O, LSE


def block_mask_dense(row_ptr, col_idx, b: int, h: int, n: int) -> np.ndarray:
    """CSR -> boolean block mask [b, h, n, n]."""
    M = np.zeros((b * h * n, n), dtype=bool)
    for r in range(b * h * n):
        M[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return M.reshape(b, h, n, n)


def masked_dense_attn(qt, kt, vt, row_ptr, col_idx, N: int, B: int, scale: float):
    """Second formulation: full token-level logits over the real tokens with -inf outside the
    selected blocks, then a row softmax (small grids only)."""
    def f64(x):
        x = np.asarray(x)
        return widen_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64, copy=False)
    qt, kt, vt = f64(qt), f64(kt), f64(vt)
    b, h, Npad, D = qt.shape
    n = num_blocks(N, B)
    Mb = block_mask_dense(row_ptr, col_idx, b, h, n)
    tok_blk = np.arange(N) // B
    O = np.full((b, h, Npad, D), np.nan)
    LSE = np.full((b, h, Npad), np.nan)
    for bi in range(b):
        for hi in range(h):
            logits = scale * (qt[bi, hi, :N] @ kt[bi, hi, :N].T)
            allowed = Mb[bi, hi][tok_blk[:, None], tok_blk[None, :]]
            logits = np.where(allowed, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            l = e.sum(axis=1, keepdims=True)
            O[bi, hi, :N] = (e @ vt[bi, hi, :N]) / l
            LSE[bi, hi, :N] = (m + np.log(l))[:, 0]
    return O, LSE


def dense_attn_raster(q, k, v, scale: float) -> np.ndarray:
    """Plain softmax attention per head on raster [b, N, h, D] inputs (no blocks, no order)."""
    def f64(x):
        x = np.asarray(x)
        return widen_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64, copy=False)
    q, k, v = f64(q), f64(k), f64(v)
    b, N, h, D = q.shape
    O = np.empty_like(q)
    for bi in range(b):
        for hi in range(h):
            o, _ = _attend(q[bi, :, hi], k[bi, :, hi], v[bi, :, hi], scale)
            O[bi, :, hi] = o
    return O


def layer(q, k, v, T, H, W, tile, B, top_p, k_floor, scale):
    """Whole path on raster inputs: reorder -> route -> sparse attention -> inverse."""
    N = T * H * W
    qt = reorder(widen_bf16(q) if np.asarray(q).dtype == np.uint16 else q, T, H, W, tile, B)
    kt = reorder(widen_bf16(k) if np.asarray(k).dtype == np.uint16 else k, T, H, W, tile, B)
    vt = reorder(widen_bf16(v) if np.asarray(v).dtype == np.uint16 else v, T, H, W, tile, B)
    rt = route(qt, kt, N, B, top_p, k_floor, scale)
    Ot, LSE = sparse_attn(qt, kt, vt, rt.row_ptr, rt.col_idx, N, B, scale)
    return inverse_reorder(Ot, T, H, W, tile), rt, Ot, LSE
