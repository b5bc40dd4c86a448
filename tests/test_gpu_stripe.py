"""GPU tests of the static periodic-stripe masks (bsa_stripe_mask) through the C ABI, against
the oracle's reading of the PSA page's six-parameter mask, and of the attention kernel run on
them (the second workload of bsa_sparse_attn_fwd).  CSRs must be bit-identical."""

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv

from gpu_common import attn_scale, bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu

P_MIX = [(1, 0, 1, 3, -1, 10), (2, -1, 3, 1, 0, 4), (1, 0, 2, 5, 2, 7), (3, 0, 3, 2, 0, 2)]


@pytest.mark.parametrize("T,H,W,tile,B,heads,batch,params", [
    (1, 3, 5, (1, 2, 2), 64, 1, 1, [(1, 0, 1, 2, 0, 3)]),           # one (ragged) block
    (5, 2, 2, (2, 1, 2), 64, 1, 1, [(2, -1, 3, 1, 1, 2)]),
    (3, 10, 13, (2, 4, 4), 64, 4, 2, P_MIX),                         # truncated tiles, batch 2
    (21, 30, 52, (4, 4, 8), 128, 4, 1, P_MIX),                       # Wan-480p grid
    (33, 45, 80, (4, 4, 8), 128, 2, 1, [(1, 0, 1, 4, -1, 10), (2, 0, 3, 3, -1, 12)]),  # Hunyuan
], ids=["tiny1", "tiny2", "ragged_batch2", "wan480p", "hunyuan720p"])
def test_stripe_csr_matches_oracle(T, H, W, tile, B, heads, batch, params):
    grid = bsa.Grid(T, H, W, tile, B)
    print(f"[gpu] stripe {T}x{H}x{W} tile {tile} B={B} heads={heads} batch={batch} "
          f"n_blk={grid.n_blk}", flush=True)
    rp, ci, nnz = bsa.stripe_mask(params, batch, heads, 128 if B == 128 else 64, grid)
    torch.cuda.synchronize()
    ref_rp, ref_ci = O.stripe_mask(T, H, W, tile, B, params, batch=batch)
    nz = int(nnz.item())
    assert nz == ref_rp[-1]
    assert np.array_equal(rp.cpu().numpy(), ref_rp)
    assert np.array_equal(ci[:nz].cpu().numpy(), ref_ci)


@pytest.mark.parametrize("D,B", [(128, 128), (64, 64)])
def test_attention_on_stripe_mask(D, B):
    cfg = Config("stripe", 4, 12, 21, 3, D, B, (4, 4, 8) if B == 128 else (2, 4, 8), 1.0, 1,
                 71 + D)
    q, k, v = gen_qkv(cfg, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    params = P_MIX[:3]
    print(f"[gpu] attention on stripe masks D={D} B={B} n_blk={grid.n_blk}", flush=True)
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in (q, k, v))
    rp, ci, nnz = bsa.stripe_mask(params, 1, cfg.heads, D, grid)
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, sc)
    torch.cuda.synchronize()
    nz = int(nnz.item())
    rp_h, ci_h = rp.cpu().numpy().astype(np.int64), ci[:nz].cpu().numpy().astype(np.int64)
    Oref, Lref = O.sparse_attn(to_bits(q_t), to_bits(k_t), to_bits(v_t), rp_h, ci_h, cfg.N, B,
                               sc)
    N = cfg.N
    d = np.abs(bf16_f64(out_t)[:, :, :N] - Oref[:, :, :N])
    print(f"[gpu]   nnz {nz} out max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy()[:, :, :N] - Lref[:, :, :N]).max() <= 1e-3
