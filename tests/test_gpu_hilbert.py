"""GPU tests of the Hilbert-curve token order (bsa_hilbert_order and grids carrying an order
table), through the C ABI, against the oracle's reading of the DFSAttn page's reordering.

* The device-built order table equals the oracle's on cube-sized and video-shaped grids.
* The whole path under that order: reorder bit-exact both ways, masks accepted on every row,
  fp64 scores, attention within the bf16 bars; the fused reorder/pooling/E4M3 outputs and the
  stripe masks follow the order too.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from oracle import fp8 as F
from workloads import Config, gen_qkv

from fp8_support import v8_to_tokens
from gpu_common import attn_scale, bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,W", [(1, 1, 1), (8, 8, 8), (5, 6, 11), (21, 30, 52), (33, 45, 80)])
def test_order_table_matches_oracle(T, H, W):
    grid = bsa.Grid(T, H, W, (4, 4, 8), 128)
    print(f"[gpu] hilbert order {T}x{H}x{W}", flush=True)
    order = bsa.hilbert_order(grid)
    torch.cuda.synchronize()
    assert np.array_equal(order.cpu().numpy(), O.hilbert_order(T, H, W))


@pytest.mark.parametrize("D,B,tile,seed", [(128, 128, (4, 4, 8), 101), (64, 64, (2, 4, 4), 102)],
                         ids=["d128b128", "d64b64"])
def test_path_under_hilbert_order(D, B, tile, seed):
    cfg = Config("hil", 4, 12, 21, 3, D, B, tile, 0.9, 2, seed)
    q, k, v = gen_qkv(cfg, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    grid = grid.with_order(bsa.hilbert_order(grid))
    pi = O.hilbert_perm(cfg.T, cfg.H, cfg.W)
    N, n = cfg.N, grid.n_blk
    print(f"[gpu] path under hilbert order D={D} B={B} N={N} n_blk={n}", flush=True)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    q_t, qbar = bsa.reorder_pool(tq, grid)
    k_t, kbar = bsa.reorder_pool(tk, grid)
    v_t = bsa.reorder(tv, grid)
    scale = 1.0 / math.sqrt(D)
    rp, ci, nnz, S = bsa.route_pooled(qbar, kbar, grid, cfg.top_p, cfg.k_floor, scale,
                                      return_scores=True)
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, sc)
    out = bsa.reorder(out_t, grid, inverse=True)
    torch.cuda.synchronize()
    for x, t in ((q, q_t), (k, k_t), (v, v_t)):
        assert np.array_equal(to_bits(t), O.reorder(x, cfg.T, cfg.H, cfg.W, tile, B, pi=pi))
    ref = O.route(to_bits(q_t), to_bits(k_t), N, B, cfg.top_p, cfg.k_floor, scale)
    s_err = np.abs(S.cpu().numpy() - ref.scores).max(axis=-1) / np.maximum(
        np.abs(ref.scores).max(axis=-1), 1e-300)
    assert s_err.max() <= 1e-12
    nz = int(nnz.item())
    rp_h, ci_h = rp.cpu().numpy().astype(np.int64), ci[:nz].cpu().numpy().astype(np.int64)
    rep = O.check_mask(ref, rp_h, ci_h, cfg.top_p, cfg.k_floor)
    assert rep.ok, rep.failures[:5]
    Oref, Lref = O.sparse_attn(to_bits(q_t), to_bits(k_t), to_bits(v_t), rp_h, ci_h, N, B, sc)
    d = np.abs(bf16_f64(out_t)[:, :, :N] - Oref[:, :, :N])
    print(f"[gpu]   masks {rep.rows} rows, nnz {nz}; out max-abs {d.max():.3e} "
          f"mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy()[:, :, :N] - Lref[:, :, :N]).max() <= 1e-3
    assert np.array_equal(to_bits(out), O.inverse_reorder(to_bits(out_t), cfg.T, cfg.H, cfg.W,
                                                          tile, pi=pi))
    # stripe masks: block coordinates from each block's first token in this order
    params = [(1, 0, 1, 3, -1, 7), (2, 0, 3, 2, 1, 5), (1, 0, 2, 4, 0, 6)]
    srp, sci, snz = bsa.stripe_mask(params, 1, cfg.heads, D, grid)
    torch.cuda.synchronize()
    r_rp, r_ci = O.stripe_mask(cfg.T, cfg.H, cfg.W, tile, B, params, pi=pi)
    assert np.array_equal(srp.cpu().numpy(), r_rp)
    assert np.array_equal(sci[:int(snz.item())].cpu().numpy(), r_ci)


def test_fp8_quantization_under_hilbert_order():
    cfg = Config("hil8", 4, 12, 21, 2, 128, 128, (4, 4, 8), 0.9, 2, 103)
    q, _, v = gen_qkv(cfg, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    grid = grid.with_order(bsa.hilbert_order(grid))
    pi = O.hilbert_perm(cfg.T, cfg.H, cfg.W)
    _, qbar, q8, qs = bsa.reorder_pool(to_dev(q), grid, tiled=False, fp8=True)
    _, v8, vs = bsa.reorder_quantize_v(to_dev(v), grid)
    torch.cuda.synchronize()
    qt = O.reorder(q, cfg.T, cfg.H, cfg.W, cfg.tile, cfg.block, pi=pi)
    vt = O.reorder(v, cfg.T, cfg.H, cfg.W, cfg.tile, cfg.block, pi=pi)
    assert np.array_equal(qbar.cpu().numpy(), O.pool(O.widen_bf16(qt), cfg.N, cfg.block))
    rc, rs = F.quantize_rows(qt, cfg.block)
    assert np.array_equal(q8.cpu().numpy(), rc) and np.array_equal(qs.cpu().numpy(), rs)
    vc, vsr = F.quantize_v(vt, cfg.block)
    assert np.array_equal(v8_to_tokens(v8.cpu().numpy()), vc)
    assert np.array_equal(vs.cpu().numpy(), vsr)


def test_fused_gathers_under_hilbert_order_batch2():
    """The fused gathers (reorder + block means, E4M3 Q/K codes, V head maxima and codes) take
    each block's raster rows from the order table once per workgroup and the batch from the
    grid: batch 2, three heads and a 6-token last block under the Hilbert order, every output
    bit-identical to the oracle's."""
    cfgs = [Config("hilb2", 3, 10, 13, 3, 128, 128, (4, 4, 8), 0.9, 2, 131 + 7 * i)
            for i in range(2)]
    parts = [gen_qkv(c, gains=np.full(c.heads, 1.5)) for c in cfgs]
    q = np.concatenate([p[0] for p in parts], axis=0)
    v = np.concatenate([p[2] for p in parts], axis=0)
    cfg = cfgs[0]
    assert cfg.N % cfg.block == 6
    grid = grid_of(cfg).with_order(bsa.hilbert_order(grid_of(cfg)))
    pi = O.hilbert_perm(cfg.T, cfg.H, cfg.W)
    print(f"[gpu] fused gathers under hilbert order batch=2 heads=3 N={cfg.N}", flush=True)
    tq, tv = to_dev(q), to_dev(v)
    q_t, qbar = bsa.reorder_pool(tq, grid)
    _, qbar8, q8, qs = bsa.reorder_pool(tq, grid, tiled=False, fp8=True)
    v_t, v8, vs = bsa.reorder_quantize_v(tv, grid, tiled=True)
    torch.cuda.synchronize()
    qt = O.reorder(q, cfg.T, cfg.H, cfg.W, cfg.tile, cfg.block, pi=pi)
    vt = O.reorder(v, cfg.T, cfg.H, cfg.W, cfg.tile, cfg.block, pi=pi)
    assert np.array_equal(to_bits(q_t), qt) and np.array_equal(to_bits(v_t), vt)
    ref_bar = O.pool(O.widen_bf16(qt), cfg.N, cfg.block)
    assert np.array_equal(qbar.cpu().numpy(), ref_bar)
    assert np.array_equal(qbar8.cpu().numpy(), ref_bar)
    rc, rs = F.quantize_rows(qt, cfg.block)
    assert np.array_equal(q8.cpu().numpy(), rc) and np.array_equal(qs.cpu().numpy(), rs)
    vc, vsr = F.quantize_v(vt, cfg.block)
    assert np.array_equal(v8_to_tokens(v8.cpu().numpy()), vc)
    assert np.array_equal(vs.cpu().numpy(), vsr)
