"""Shared helpers of the GPU parity tests: move seeded bf16 inputs to the device, run the
HIP path through the C ABI binding, bring results back as NumPy."""
import math

import numpy as np
import torch

import block_sparse_attention_gather_amd as bsa


def grid_of(cfg) -> bsa.Grid:
    return bsa.Grid(cfg.T, cfg.H, cfg.W, tuple(cfg.tile), cfg.block)


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 tensor on cuda:0 (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def attn_scale(D: int) -> float:
    """The fp32 softmax scale the kernels receive, as an exact fp64 value."""
    return float(np.float32(1.0 / math.sqrt(D)))


def run_path(grid: bsa.Grid, q, k, v, top_p, k_floor, want_scores=True):
    """Whole HIP path on raster bf16 bits -> dict of NumPy results."""
    D = q.shape[-1]
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    q_t = bsa.reorder(tq, grid)
    k_t = bsa.reorder(tk, grid)
    v_t = bsa.reorder(tv, grid)
    res = bsa.score_and_route(q_t, k_t, grid, top_p, k_floor, 1.0 / math.sqrt(D),
                              return_scores=want_scores)
    row_ptr, col_idx, nnz = res[:3]
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, row_ptr, col_idx, grid, attn_scale(D))
    out = bsa.reorder(out_t, grid, inverse=True)
    torch.cuda.synchronize()
    nz = int(nnz.item())
    return dict(
        q_t=to_bits(q_t), k_t=to_bits(k_t), v_t=to_bits(v_t),
        row_ptr=row_ptr.cpu().numpy().astype(np.int64),
        col_idx=col_idx[:nz].cpu().numpy().astype(np.int64), nnz=nz,
        scores=res[3].cpu().numpy() if want_scores else None,
        out_t=bf16_f64(out_t), lse=lse.cpu().numpy().astype(np.float64),
        out=bf16_f64(out), out_bits=to_bits(out_t))
