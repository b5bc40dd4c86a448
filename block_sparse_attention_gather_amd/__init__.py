"""Python binding of libbsa: training-free block-sparse video attention on MI355X (gfx950).

Argument marshalling only.  Every step runs in the HIP kernels of libbsa.so; PyTorch tensors
supply device memory and the current HIP stream.  There is no fallback: if the library is not
built, or a tensor is not on a GPU, the calls raise.

    grid = Grid(T=21, H=30, W=52, tile=(4, 4, 8), block=128)
    q_t = reorder(q, grid)                        # [b, N, h, D] -> [b, h, Npad, D]
    row_ptr, col_idx, nnz = score_and_route(q_t, k_t, grid, top_p=0.9, k_floor=8)
    out_t, lse = sparse_attn_fwd(q_t, k_t, v_t, row_ptr, col_idx, grid)
    out = reorder(out_t, grid, inverse=True)      # [b, h, Npad, D] -> [b, N, h, D]

    out, row_ptr, col_idx, nnz = layer(q, k, v, grid, 0.9, 8)   # the same, fused as benchmarked
    grid_h = grid.with_order(hilbert_order(grid))                # Hilbert-curve token order
    MaskReuse(2).layer(q, k, v, grid, 0.9, 8)                    # route every 2nd step only
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsa.so")
TRACE_LIB_PATH = os.path.join(_PKG, "libbsa_trace.so")   # debug build with bsa_trace_read

BSA_OK = 0
_STATUS = {-1: "BSA_ERR_INVALID_ARG", -2: "BSA_ERR_UNSUPPORTED", -3: "BSA_ERR_WORKSPACE",
           -4: "BSA_ERR_HIP"}


class BsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class _Grid(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("tile_t", ctypes.c_int32), ("tile_h", ctypes.c_int32),
                ("tile_w", ctypes.c_int32), ("block", ctypes.c_int32),
                ("order", ctypes.c_void_p)]


class _Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32)]


@dataclass(frozen=True)
class Grid:
    """Latent grid T x H x W, 3D tile extent and block size (tokens per block); `order`
    (optional int32 GPU tensor of N entries, e.g. hilbert_order(grid)) replaces the 3D-tile
    token order."""
    T: int
    H: int
    W: int
    tile: Tuple[int, int, int]
    block: int
    order: Optional[object] = field(default=None, compare=False, hash=False, repr=False)

    def with_order(self, order) -> "Grid":
        return Grid(self.T, self.H, self.W, tuple(self.tile), self.block, order)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def n_blk(self) -> int:
        return -(-self.N // self.block)

    @property
    def Npad(self) -> int:
        return self.n_blk * self.block

    def _c(self) -> _Grid:
        return _Grid(self.T, self.H, self.W, self.tile[0], self.tile[1], self.tile[2],
                     self.block, None if self.order is None else self.order.data_ptr())


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libbsa.so not built at {LIB_PATH}; run "
                          "`python -m block_sparse_attention_gather_amd.build`")
    # torch first: it loads its own HIP runtime, and libbsa's HIP dependency must bind to that
    # same runtime (a second runtime loaded ahead of it finds no device)
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, F64, F32, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_float,
                            ctypes.c_size_t)
    G, S = ctypes.POINTER(_Grid), ctypes.POINTER(_Shape)
    sigs = {
        "bsa_num_blocks": (I32, [G]),
        "bsa_hilbert_order_workspace_bytes": (SZ, [G]),
        "bsa_hilbert_order": (I32, [G, P, P, SZ, P]),
        "bsa_padded_len": (I32, [G]),
        "bsa_reorder": (I32, [P, P, S, G, I32, P]),
        "bsa_reorder_pool": (I32, [P, P, P, P, P, S, G, P]),
        "bsa_reorder_quantize_v": (I32, [P, P, P, P, S, G, P]),
        "bsa_route_workspace_bytes": (SZ, [S, G]),
        "bsa_score_and_route": (I32, [P, P, S, G, F64, I32, F64, P, P, P, P, P, SZ, P]),
        "bsa_route_pooled": (I32, [P, P, S, G, F64, I32, F64, P, P, P, P, P, SZ, P]),
        "bsa_stripe_workspace_bytes": (SZ, [S, G]),
        "bsa_stripe_mask": (I32, [P, S, G, P, P, P, P, SZ, P]),
        "bsa_attn_workspace_bytes": (SZ, [S, G]),
        "bsa_quantize_fp8": (I32, [P, P, P, I32, S, G, P]),
        "bsa_attn_fp8_workspace_bytes": (SZ, [S, G]),
        "bsa_sparse_attn_fwd_fp8": (I32, [P, P, P, P, P, P, P, P, S, G, F32, I32, P, P, P, SZ,
                                           P]),
        "bsa_sparse_attn_fwd": (I32, [P, P, P, P, P, S, G, F32, P, P, P, SZ, P]),
        "bsa_sparse_attn_fwd_noalloc": (I32, [P, P, P, P, P, S, G, F32, P, P, P]),
        "bsa_last_error": (ctypes.c_char_p, []),
        "bsa_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def load_library(path: str):
    """Route every later call through another build of libbsa (e.g. TRACE_LIB_PATH)."""
    global _lib, LIB_PATH
    LIB_PATH = path
    _lib = None
    return _load()


# one record per attention workgroup (debug build): s_memrealtime ticks (100 MHz) at entry,
# after the last work item and at exit; s_memtime (shader clock) ticks at entry and exit;
# HW_REG_HW_ID and XCC id; items and key blocks done
TRACE_DTYPE = [("t0", "<u8"), ("t_last", "<u8"), ("t_end", "<u8"), ("c0", "<u8"),
               ("c_end", "<u8"), ("hw_id", "<u4"), ("xcc", "<u4"), ("items", "<i4"),
               ("blocks", "<i4")]
TRACE_MAX = 8192


def trace_read(count: int = TRACE_MAX):
    """Workgroup records of the latest attention launch (needs libbsa_trace.so loaded).
    Synchronous.  Returns a NumPy structured array with the records that were written."""
    import numpy as np
    lib = _load()
    if not hasattr(lib, "bsa_trace_read"):
        raise BsaError(-1, f"{LIB_PATH} is not a trace build")
    fn = lib.bsa_trace_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    buf = np.zeros(count, dtype=TRACE_DTYPE)
    rc = fn(buf.ctypes.data, count)
    if rc != 0:
        raise BsaError(-4, f"bsa_trace_read failed ({rc})")
    return buf[buf["t_end"] != 0]


def version() -> str:
    return _load().bsa_version().decode()


def _check(status: int):
    if status != BSA_OK:
        raise BsaError(status, _load().bsa_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _require(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need(t, dtype, shape, name):
    """t must be a contiguous GPU tensor of `dtype` with exactly `shape`: the C ABI sees only
    a pointer, so a smaller buffer would be written out of bounds."""
    _require(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _shape(batch, heads, D) -> _Shape:
    return _Shape(batch, heads, D)


# ---------------------------------------------------------------------------------------
def reorder(x, grid: Grid, inverse: bool = False, out=None):
    """3D-tile token permutation.  inverse=False: raster [b, N, h, D] -> tiled [b, h, Npad, D]
    (pad rows zero); inverse=True: tiled -> raster (pad rows dropped)."""
    import torch
    _require(x, torch.bfloat16, "x")
    if not inverse:
        b, N, h, D = x.shape
        if N != grid.N:
            raise ValueError(f"x has {N} tokens, grid has {grid.N}")
        shape_out = (b, h, grid.Npad, D)
    else:
        b, h, Np, D = x.shape
        if Np != grid.Npad:
            raise ValueError(f"x has {Np} rows, grid pads to {grid.Npad}")
        shape_out = (b, grid.N, h, D)
    if out is None:
        out = torch.empty(shape_out, dtype=x.dtype, device=x.device)
    _require(out, torch.bfloat16, "out")
    if tuple(out.shape) != shape_out:
        raise ValueError(f"out must have shape {shape_out}")
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_reorder(x.data_ptr(), out.data_ptr(), ctypes.byref(s), ctypes.byref(g),
                               int(bool(inverse)), _stream(x)))
    return out


def reorder_pool(x, grid: Grid, out=None, pooled=None, tiled: bool = True, fp8: bool = False,
                 x8=None, x8_scales=None, pool: bool = True):
    """Forward reorder plus the per-block means routing pools, in one pass over raster
    x [b, N, h, D] bf16 -> (tiled [b, h, Npad, D] bf16 or None, pooled [b, h, n_blk, D] fp64)
    and, with fp8=True, also the E4M3 codes [b, h, Npad, D] and per-block scales
    [b, h, n_blk] of quantize_fp8 -> (tiled, pooled, x8, x8_scales).  tiled=False skips the
    bf16 output; pool=False skips the block means (pooled is then None; needs another output)."""
    import torch
    _require(x, torch.bfloat16, "x")
    b, N, h, D = x.shape
    if N != grid.N:
        raise ValueError(f"x has {N} tokens, grid has {grid.N}")
    dev = x.device
    if tiled and out is None:
        out = torch.empty((b, h, grid.Npad, D), dtype=x.dtype, device=dev)
    if out is not None:
        _require(out, torch.bfloat16, "out")
        if tuple(out.shape) != (b, h, grid.Npad, D):
            raise ValueError(f"out must have shape {(b, h, grid.Npad, D)}")
    if not pool:
        pooled = None
    else:
        if pooled is None:
            pooled = torch.empty((b, h, grid.n_blk, D), dtype=torch.float64, device=dev)
        _require(pooled, torch.float64, "pooled")
        if tuple(pooled.shape) != (b, h, grid.n_blk, D):
            raise ValueError(f"pooled must have shape {(b, h, grid.n_blk, D)}")
    if fp8:
        if x8 is None:
            x8 = torch.empty((b, h, grid.Npad, D), dtype=torch.uint8, device=dev)
        if x8_scales is None:
            x8_scales = torch.empty((b, h, grid.n_blk), dtype=torch.float32, device=dev)
        _need(x8, torch.uint8, (b, h, grid.Npad, D), "x8")
        _need(x8_scales, torch.float32, (b, h, grid.n_blk), "x8_scales")
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_reorder_pool(x.data_ptr(), _ptr(out), _ptr(pooled),
                                    _ptr(x8) if fp8 else None,
                                    _ptr(x8_scales) if fp8 else None,
                                    ctypes.byref(s), ctypes.byref(g), _stream(x)))
    if fp8:
        return out, pooled, x8, x8_scales
    return out, pooled


def reorder_quantize_v(x, grid: Grid, out=None, tiled: bool = False, v8=None, v_scales=None):
    """Raster V [b, N, h, 128] bf16 -> (tiled bf16 or None, E4M3 codes [b, h, n_blk, 128, 128],
    per-head scales [b, h]) as reorder + quantize_fp8(v_layout=True)."""
    import torch
    _require(x, torch.bfloat16, "x")
    b, N, h, D = x.shape
    if N != grid.N:
        raise ValueError(f"x has {N} tokens, grid has {grid.N}")
    dev = x.device
    if tiled and out is None:
        out = torch.empty((b, h, grid.Npad, D), dtype=x.dtype, device=dev)
    if out is not None:
        _need(out, torch.bfloat16, (b, h, grid.Npad, D), "out")
    if v8 is None:
        v8 = torch.empty((b, h, grid.n_blk, D, grid.block), dtype=torch.uint8, device=dev)
    if v_scales is None:
        v_scales = torch.empty((b, h), dtype=torch.float32, device=dev)
    _need(v8, torch.uint8, (b, h, grid.n_blk, D, grid.block), "v8")
    _need(v_scales, torch.float32, (b, h), "v_scales")
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_reorder_quantize_v(x.data_ptr(), _ptr(out), v8.data_ptr(),
                                          v_scales.data_ptr(), ctypes.byref(s), ctypes.byref(g),
                                          _stream(x)))
    return out, v8, v_scales


def hilbert_order(grid: Grid, device="cuda:0"):
    """Hilbert-curve token order of the grid as an int32 tensor of N entries (order[p] = raster
    token at position p); use it with grid.with_order(...)."""
    import torch
    g = grid._c()
    n = int(_load().bsa_hilbert_order_workspace_bytes(ctypes.byref(g)))
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    order = torch.empty(grid.N, dtype=torch.int32, device=device)
    _check(_load().bsa_hilbert_order(ctypes.byref(g), order.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream(order)))
    return order


def route_workspace_bytes(batch, heads, D, grid: Grid) -> int:
    g, s = grid._c(), _shape(batch, heads, D)
    return int(_load().bsa_route_workspace_bytes(ctypes.byref(s), ctypes.byref(g)))


def attn_workspace_bytes(batch, heads, D, grid: Grid) -> int:
    g, s = grid._c(), _shape(batch, heads, D)
    n = int(_load().bsa_attn_workspace_bytes(ctypes.byref(s), ctypes.byref(g)))
    if n == 0:
        _check(-4 if not _load().bsa_last_error() else -1)
    return n


def _route_outputs(b, h, D, grid, dev, return_scores, workspace, row_ptr, col_idx, nnz):
    import torch
    rows = b * h * grid.n_blk
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(rows * grid.n_blk, dtype=torch.int32, device=dev)
    if nnz is None:
        nnz = torch.empty(1, dtype=torch.int32, device=dev)
    for t, n, size in ((row_ptr, "row_ptr", rows + 1), (col_idx, "col_idx", rows * grid.n_blk),
                       (nnz, "nnz", 1)):
        _require(t, torch.int32, n)
        if t.numel() < size:
            raise ValueError(f"{n} needs {size} int32 entries")
    scores = (torch.empty((b, h, grid.n_blk, grid.n_blk), dtype=torch.float64, device=dev)
              if return_scores else None)
    need = route_workspace_bytes(b, h, D, grid)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    return scores, workspace, row_ptr, col_idx, nnz


def score_and_route(q_t, k_t, grid: Grid, top_p: float, k_floor: int,
                    scale: Optional[float] = None, return_scores: bool = False,
                    workspace=None, row_ptr=None, col_idx=None, nnz=None):
    """Pooled block scores and Top-p / Top-k routing -> (row_ptr, col_idx, nnz[, scores]).

    col_idx has the worst-case capacity rows * n_blk; its first nnz entries are the CSR
    columns.  nnz stays on the device (a 1-element int32 tensor)."""
    import torch
    _require(q_t, torch.bfloat16, "q_t")
    _require(k_t, torch.bfloat16, "k_t")
    b, h, Np, D = q_t.shape
    if tuple(k_t.shape) != (b, h, Np, D) or Np != grid.Npad:
        raise ValueError("q_t/k_t must both be [b, h, Npad, D] for this grid")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    scores, workspace, row_ptr, col_idx, nnz = _route_outputs(
        b, h, D, grid, q_t.device, return_scores, workspace, row_ptr, col_idx, nnz)
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_score_and_route(
        q_t.data_ptr(), k_t.data_ptr(), ctypes.byref(s), ctypes.byref(g), float(top_p),
        int(k_floor), scale, row_ptr.data_ptr(), col_idx.data_ptr(), nnz.data_ptr(),
        _ptr(scores), workspace.data_ptr(), workspace.numel(), _stream(q_t)))
    if return_scores:
        return row_ptr, col_idx, nnz, scores
    return row_ptr, col_idx, nnz


def route_pooled(qbar, kbar, grid: Grid, top_p: float, k_floor: int,
                 scale: Optional[float] = None, return_scores: bool = False,
                 workspace=None, row_ptr=None, col_idx=None, nnz=None):
    """score_and_route from the block means reorder_pool returns ([b, h, n_blk, D] fp64);
    same outputs as score_and_route on the tiled Q and K."""
    import torch
    _require(qbar, torch.float64, "qbar")
    _require(kbar, torch.float64, "kbar")
    b, h, n, D = qbar.shape
    if tuple(kbar.shape) != (b, h, n, D) or n != grid.n_blk:
        raise ValueError("qbar/kbar must both be [b, h, n_blk, D] for this grid")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    scores, workspace, row_ptr, col_idx, nnz = _route_outputs(
        b, h, D, grid, qbar.device, return_scores, workspace, row_ptr, col_idx, nnz)
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_route_pooled(
        qbar.data_ptr(), kbar.data_ptr(), ctypes.byref(s), ctypes.byref(g), float(top_p),
        int(k_floor), scale, row_ptr.data_ptr(), col_idx.data_ptr(), nnz.data_ptr(),
        _ptr(scores), workspace.data_ptr(), workspace.numel(), _stream(qbar)))
    if return_scores:
        return row_ptr, col_idx, nnz, scores
    return row_ptr, col_idx, nnz


def stripe_mask(params, batch: int, heads: int, D: int, grid: Grid, device="cuda:0",
                workspace=None, row_ptr=None, col_idx=None, nnz=None):
    """Static periodic-stripe masks -> CSR (row_ptr, col_idx, nnz) in the routing's format.

    params: one (Tw, To, Ts, Sw, So, Ss) for every head, or a list of `heads` of them."""
    import torch
    p = list(params)
    if p and not isinstance(p[0], (tuple, list)):
        p = [tuple(p)] * heads
    if len(p) != heads or any(len(x) != 6 for x in p):
        raise ValueError("params: one (Tw, To, Ts, Sw, So, Ss) per head")
    arr = (ctypes.c_int32 * (6 * heads))(*[int(v) for x in p for v in x])
    dev = torch.device(device)
    rows = batch * heads * grid.n_blk
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    if col_idx is None:
        col_idx = torch.empty(rows * grid.n_blk, dtype=torch.int32, device=dev)
    if nnz is None:
        nnz = torch.empty(1, dtype=torch.int32, device=dev)
    for t, n, size in ((row_ptr, "row_ptr", rows + 1), (col_idx, "col_idx", rows * grid.n_blk),
                       (nnz, "nnz", 1)):
        _require(t, torch.int32, n)
        if t.numel() < size:
            raise ValueError(f"{n} needs {size} int32 entries")
    g, s = grid._c(), _shape(batch, heads, D)
    if workspace is None:
        need = int(_load().bsa_stripe_workspace_bytes(ctypes.byref(s), ctypes.byref(g)))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(_load().bsa_stripe_mask(arr, ctypes.byref(s), ctypes.byref(g), row_ptr.data_ptr(),
                                   col_idx.data_ptr(), nnz.data_ptr(), workspace.data_ptr(),
                                   workspace.numel(), _stream(row_ptr)))
    return row_ptr, col_idx, nnz


def sparse_attn_fwd(q_t, k_t, v_t, row_ptr, col_idx, grid: Grid,
                    scale: Optional[float] = None, return_lse: bool = True, out=None,
                    lse=None, workspace=None):
    """Exact attention over the CSR-selected key blocks -> (out_t [b, h, Npad, D] bf16,
    lse [b, h, Npad] fp32 or None)."""
    import torch
    for t, n in ((q_t, "q_t"), (k_t, "k_t"), (v_t, "v_t")):
        _require(t, torch.bfloat16, n)
    _require(row_ptr, torch.int32, "row_ptr")
    _require(col_idx, torch.int32, "col_idx")
    b, h, Np, D = q_t.shape
    if tuple(k_t.shape) != (b, h, Np, D) or tuple(v_t.shape) != (b, h, Np, D):
        raise ValueError("q_t/k_t/v_t must have the same shape")
    if Np != grid.Npad:
        raise ValueError(f"tiled tensors need {grid.Npad} rows")
    if row_ptr.numel() != b * h * grid.n_blk + 1:
        raise ValueError("row_ptr must have rows + 1 entries")
    if col_idx.dim() != 1 or col_idx.numel() < 1:
        raise ValueError("col_idx must be a 1-D tensor holding at least row_ptr[rows] entries")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q_t.device
    if out is None:
        out = torch.empty_like(q_t)
    _need(out, torch.bfloat16, (b, h, Np, D), "out")
    if return_lse and lse is None:
        lse = torch.empty((b, h, Np), dtype=torch.float32, device=dev)
    if return_lse:
        _need(lse, torch.float32, (b, h, Np), "lse")
    if workspace is None:
        workspace = torch.empty(attn_workspace_bytes(b, h, D, grid), dtype=torch.uint8,
                                device=dev)
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_sparse_attn_fwd(
        q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), row_ptr.data_ptr(), col_idx.data_ptr(),
        ctypes.byref(s), ctypes.byref(g), scale, out.data_ptr(),
        _ptr(lse) if return_lse else None, workspace.data_ptr(), workspace.numel(),
        _stream(q_t)))
    return out, (lse if return_lse else None)


def sparse_attn_fwd_noalloc(q_t, k_t, v_t, row_ptr, col_idx, grid: Grid, out, lse=None,
                            scale: Optional[float] = None):
    """sparse_attn_fwd for callers that cannot allocate: the caller passes the output (and
    optionally lse) buffers, and the library works in its static per-device scratch instead
    of a workspace.  Same result as sparse_attn_fwd, bit for bit.  Calls that overlap on one
    device share that scratch and must be ordered.  Returns (out, lse)."""
    import torch
    for t, n in ((q_t, "q_t"), (k_t, "k_t"), (v_t, "v_t")):
        _require(t, torch.bfloat16, n)
    _require(row_ptr, torch.int32, "row_ptr")
    _require(col_idx, torch.int32, "col_idx")
    b, h, Np, D = q_t.shape
    if tuple(k_t.shape) != (b, h, Np, D) or tuple(v_t.shape) != (b, h, Np, D):
        raise ValueError("q_t/k_t/v_t must have the same shape")
    if Np != grid.Npad:
        raise ValueError(f"tiled tensors need {grid.Npad} rows")
    if row_ptr.numel() != b * h * grid.n_blk + 1:
        raise ValueError("row_ptr must have rows + 1 entries")
    if col_idx.dim() != 1 or col_idx.numel() < 1:
        raise ValueError("col_idx must be a 1-D tensor holding at least row_ptr[rows] entries")
    _need(out, torch.bfloat16, (b, h, Np, D), "out")
    if lse is not None:
        _need(lse, torch.float32, (b, h, Np), "lse")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_sparse_attn_fwd_noalloc(
        q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), row_ptr.data_ptr(), col_idx.data_ptr(),
        ctypes.byref(s), ctypes.byref(g), scale, out.data_ptr(), _ptr(lse), _stream(q_t)))
    return out, lse


def quantize_fp8(x_t, grid: Grid, v_layout: bool = False, out=None, scales=None):
    """E4M3 codes of a tiled bf16 tensor [b, h, Npad, 128] -> (codes uint8, scales fp32).

    v_layout=False (Q, K): codes [b, h, Npad, 128], one scale per 128-token block [b, h, n_blk];
    v_layout=True (V): codes [b, h, n_blk, 128, 128] (blocks transposed, keys in the FP8
    kernel's lane order), one scale per (batch, head) [b, h]."""
    import torch
    _require(x_t, torch.bfloat16, "x_t")
    b, h, Np, D = x_t.shape
    if Np != grid.Npad:
        raise ValueError(f"x_t needs {grid.Npad} rows")
    shape_o = (b, h, grid.n_blk, D, grid.block) if v_layout else (b, h, Np, D)
    shape_s = (b, h) if v_layout else (b, h, grid.n_blk)
    if out is None:
        out = torch.empty(shape_o, dtype=torch.uint8, device=x_t.device)
    if scales is None:
        scales = torch.empty(shape_s, dtype=torch.float32, device=x_t.device)
    _require(out, torch.uint8, "out")
    _require(scales, torch.float32, "scales")
    if tuple(out.shape) != shape_o or tuple(scales.shape) != shape_s:
        raise ValueError(f"out must be {shape_o} and scales {shape_s}")
    g, s = grid._c(), _shape(b, h, D)
    _check(_load().bsa_quantize_fp8(x_t.data_ptr(), out.data_ptr(), scales.data_ptr(),
                                    int(bool(v_layout)), ctypes.byref(s), ctypes.byref(g),
                                    _stream(x_t)))
    return out, scales


def sparse_attn_fwd_fp8(q8, q_scale, k8, k_scale, v8, v_scale, row_ptr, col_idx, grid: Grid,
                        scale: Optional[float] = None, out=None, lse=None, workspace=None,
                        return_lse: bool = True, expcast: bool = False):
    """FP8 attention over quantize_fp8 outputs -> (out_t [b, h, Npad, 128] bf16, lse).
    expcast=True casts the probabilities with ExpCast (one FMA, no exponential)."""
    import torch
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _require(t, torch.uint8, n)
    for t, n in ((q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _require(t, torch.float32, n)
    _require(row_ptr, torch.int32, "row_ptr")
    _require(col_idx, torch.int32, "col_idx")
    b, h, Np, D = q8.shape
    if tuple(k8.shape) != (b, h, Np, D) or tuple(v8.shape) != (b, h, grid.n_blk, D, grid.block):
        raise ValueError("k8 must match q8, v8 must be [b, h, n_blk, D, B]")
    if row_ptr.numel() != b * h * grid.n_blk + 1:
        raise ValueError("row_ptr must have rows + 1 entries")
    if col_idx.dim() != 1 or col_idx.numel() < 1:
        raise ValueError("col_idx must be a 1-D tensor holding at least row_ptr[rows] entries")
    if Np != grid.Npad:
        raise ValueError(f"q8/k8 need {grid.Npad} rows")
    _need(q_scale, torch.float32, (b, h, grid.n_blk), "q_scale")
    _need(k_scale, torch.float32, (b, h, grid.n_blk), "k_scale")
    _need(v_scale, torch.float32, (b, h), "v_scale")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dev = q8.device
    if out is None:
        out = torch.empty((b, h, Np, D), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, (b, h, Np, D), "out")
    if return_lse and lse is None:
        lse = torch.empty((b, h, Np), dtype=torch.float32, device=dev)
    if return_lse:
        _need(lse, torch.float32, (b, h, Np), "lse")
    g, s = grid._c(), _shape(b, h, D)
    if workspace is None:
        n = int(_load().bsa_attn_fp8_workspace_bytes(ctypes.byref(s), ctypes.byref(g)))
        if n == 0:
            _check(-2)
        workspace = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(_load().bsa_sparse_attn_fwd_fp8(
        q8.data_ptr(), q_scale.data_ptr(), k8.data_ptr(), k_scale.data_ptr(), v8.data_ptr(),
        v_scale.data_ptr(), row_ptr.data_ptr(), col_idx.data_ptr(), ctypes.byref(s),
        ctypes.byref(g), scale, int(bool(expcast)), out.data_ptr(),
        _ptr(lse) if return_lse else None,
        workspace.data_ptr(), workspace.numel(), _stream(q8)))
    return out, (lse if return_lse else None)


def layer(q, k, v, grid: Grid, top_p: float, k_floor: int, scale: Optional[float] = None,
          mask=None):
    """Whole path on raster [b, N, h, D] bf16 inputs -> (out [b, N, h, D], row_ptr, col_idx,
    nnz).  mask = (row_ptr, col_idx, nnz) of an earlier call on the same grid and shape reuses
    that CSR: the block pooling and the routing are skipped and only the reorders and the
    attention run (mask reuse across denoising steps)."""
    if mask is None:
        q_t, qbar = reorder_pool(q, grid)
        k_t, kbar = reorder_pool(k, grid)
        v_t = reorder(v, grid)
        row_ptr, col_idx, nnz = route_pooled(qbar, kbar, grid, top_p, k_floor, scale)
    else:
        row_ptr, col_idx, nnz = mask
        b, _, h, _ = q.shape
        if row_ptr.numel() != b * h * grid.n_blk + 1:
            raise ValueError(f"mask row_ptr has {row_ptr.numel()} entries, this call needs "
                             f"{b * h * grid.n_blk + 1}")
        q_t, k_t, v_t = reorder(q, grid), reorder(k, grid), reorder(v, grid)
    out_t, _ = sparse_attn_fwd(q_t, k_t, v_t, row_ptr, col_idx, grid, scale,
                               return_lse=False)
    return reorder(out_t, grid, inverse=True), row_ptr, col_idx, nnz


class MaskReuse:
    """Mask reuse across denoising steps (the DFSAttn page, abstract, caches sparse masks; read
    here as reuse across the steps of a layer): the first call of every `interval` consecutive
    calls routes, the others reuse its CSR.  interval = 1 routes every call.  Host-side bookkeeping only; each call runs
    `layer`."""

    def __init__(self, interval: int):
        if int(interval) < 1:
            raise ValueError("interval must be >= 1")
        self.interval = int(interval)
        self.calls = 0
        self.mask = None

    def layer(self, q, k, v, grid: Grid, top_p: float, k_floor: int,
              scale: Optional[float] = None):
        """-> (out, routed): `routed` says whether this call computed a new mask."""
        routed = self.mask is None or self.calls % self.interval == 0
        out, row_ptr, col_idx, nnz = layer(q, k, v, grid, top_p, k_floor, scale,
                                           mask=None if routed else self.mask)
        self.mask = (row_ptr, col_idx, nnz)
        self.calls += 1
        return out, routed
