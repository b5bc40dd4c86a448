"""GPU tests of the fused forward path (bsa_reorder_pool + bsa_route_pooled) through the C ABI.

* The tiled output of bsa_reorder_pool is bit-identical to the oracle's token permutation and
  to bsa_reorder; its block means are bit-identical to the oracle's pooling (exact fp64 sums
  of bf16 values divided by the block's real-token count), for batch > 1, a ragged last block,
  truncated tiles on every axis and each (head_dim, block) kernel.
* bsa_route_pooled on those means returns exactly the CSR and the block scores of
  bsa_score_and_route on the tiled Q and K.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv

from gpu_common import grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,B,tile,grid3,heads,batch,seed", [
    (128, 128, (4, 4, 8), (5, 10, 21), 3, 2, 61),
    (64, 64, (2, 4, 4), (3, 10, 13), 2, 3, 62),
    (128, 64, (4, 4, 4), (4, 12, 20), 2, 1, 63),
    (64, 128, (4, 4, 8), (4, 12, 21), 2, 2, 64),
], ids=["d128b128_batch2", "d64b64_batch3", "d128b64", "d64b128_batch2"])
def test_reorder_pool_and_route_pooled(D, B, tile, grid3, heads, batch, seed):
    T, H, W = grid3
    cfgs = [Config("fused", T, H, W, heads, D, B, tile, 0.9, 2, seed + 10 * i)
            for i in range(batch)]
    qs, ks = [], []
    for c in cfgs:
        q, k, _ = gen_qkv(c, gains=np.full(heads, 1.5))
        qs.append(q)
        ks.append(k)
    q = np.concatenate(qs, axis=0)                # [batch, N, heads, D] bf16 bits
    k = np.concatenate(ks, axis=0)
    cfg = cfgs[0]
    grid = grid_of(cfg)
    print(f"[gpu] reorder_pool D={D} B={B} batch={batch} heads={heads} N={cfg.N} "
          f"n_blk={grid.n_blk}", flush=True)
    tq, tk = to_dev(q), to_dev(k)
    q_t, qbar = bsa.reorder_pool(tq, grid)
    k_t, kbar = bsa.reorder_pool(tk, grid)
    q_t_plain = bsa.reorder(tq, grid)
    torch.cuda.synchronize()
    ref_t = O.reorder(q, T, H, W, tile, B)
    assert np.array_equal(to_bits(q_t), ref_t)
    assert torch.equal(q_t.view(torch.int16), q_t_plain.view(torch.int16))
    ref_bar = O.pool(O.widen_bf16(ref_t), cfg.N, B)
    assert np.array_equal(qbar.cpu().numpy(), ref_bar)
    assert np.array_equal(kbar.cpu().numpy(),
                          O.pool(O.widen_bf16(O.reorder(k, T, H, W, tile, B)), cfg.N, B))
    # routing from the means == routing from the tiled tensors
    a = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor, return_scores=True)
    b = bsa.route_pooled(qbar, kbar, grid, cfg.top_p, cfg.k_floor, return_scores=True)
    torch.cuda.synchronize()
    nz = int(a[2].item())
    assert int(b[2].item()) == nz
    assert torch.equal(a[0], b[0])
    assert torch.equal(a[1][:nz], b[1][:nz])
    assert torch.equal(a[3], b[3])
