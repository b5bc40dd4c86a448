"""GPU routing on long rows, through the C ABI binding, against the fp64 oracle.

Rows of up to 2048 blocks take the MFMA score kernel and the one-wavefront-per-row sort; longer
rows take the workgroup LDS sort.  Both are checked at their edges: exactly 2048 blocks (the
largest wavefront sort), and 2142 blocks with truncated tiles on every axis and a ragged last
block.  The CSR must be the same whether the block scores go to the caller's buffer or stay in
the workspace."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv

from gpu_common import grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,W,seed", [(32, 64, 64, 51), (33, 62, 67, 52)],
                         ids=["n2048_wave", "n2142_lds"])
def test_route_long_rows(T, H, W, seed):
    cfg = Config("long", T, H, W, 1, 64, 64, (4, 4, 4), 0.9, 4, seed)
    q, k, _ = gen_qkv(cfg, gains=np.full(1, 1.5))
    grid = grid_of(cfg)
    n = grid.n_blk
    print(f"[gpu] route long rows: N={cfg.N} n_blk={n}", flush=True)
    q_t = bsa.reorder(to_dev(q), grid)
    k_t = bsa.reorder(to_dev(k), grid)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    rp, ci, nnz, S = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor, scale,
                                         return_scores=True)
    rp2, ci2, nnz2 = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor, scale,
                                         return_scores=False)[:3]
    torch.cuda.synchronize()
    nz = int(nnz.item())
    assert int(nnz2.item()) == nz
    assert torch.equal(rp, rp2) and torch.equal(ci[:nz], ci2[:nz])
    ref = O.route(to_bits(q_t), to_bits(k_t), cfg.N, cfg.block, cfg.top_p, cfg.k_floor, scale)
    s = S.cpu().numpy()
    s_err = np.abs(s - ref.scores).max(axis=-1) / np.maximum(np.abs(ref.scores).max(axis=-1),
                                                             1e-300)
    assert s_err.max() <= 1e-12, s_err.max()
    rep = O.check_mask(ref, rp.cpu().numpy(), ci[:nz].cpu().numpy(), cfg.top_p, cfg.k_floor)
    print(f"[gpu]   mask rows {rep.rows}: exact {rep.exact} tie {rep.tie} count {rep.count} "
          f"nnz {nz}", flush=True)
    assert rep.ok, rep.failures[:5]
