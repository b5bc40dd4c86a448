"""GPU tests of the FP8 (E4M3) path through the C ABI, against the oracle's FP8 reading.

* Quantization: the codes and scales of bsa_quantize_fp8 are bit-identical to the oracle's
  (per-block Q/K, per-head V, compared token-major), including an all-zero block and a ragged tail.
* Attention: bsa_sparse_attn_fwd_fp8 against the exact fp64 attention over the dequantized
  inputs, per element within the bound on what casting the probabilities to E4M3 can change
  (oracle/fp8.attn_error_bound / expcast_error_bound) plus the kernel's fp32 arithmetic and
  the bf16 rounding of the output (fp8_support.fp8_out_tol); LSE within 1e-3 (plus the ExpCast
  bound on the lse).  One routed CSR and one whose rows are split and merged.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from oracle import fp8 as F
from workloads import Config, gen_qkv

from fp8_support import fp8_out_tol, v8_to_tokens
from gpu_common import attn_scale, bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _tiled(cfg, zero_block=None):
    q, k, v = gen_qkv(cfg, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in (q, k, v))
    blocks = [] if zero_block is None else (
        zero_block if isinstance(zero_block, list) else [zero_block])
    for hh, j in blocks:
        for t in (q_t, k_t):
            t[0, hh, j * cfg.block:(j + 1) * cfg.block] = 0
    return grid, q_t, k_t, v_t


def test_quantize_matches_oracle():
    cfg = Config("f8q", 4, 12, 21, 2, 128, 128, (4, 4, 8), 0.9, 2, 81)
    grid, q_t, k_t, v_t = _tiled(cfg, zero_block=(1, 3))
    print(f"[gpu] fp8 quantize N={cfg.N} n_blk={grid.n_blk}", flush=True)
    q8, qs = bsa.quantize_fp8(q_t, grid)
    v8, vs = bsa.quantize_fp8(v_t, grid, v_layout=True)
    torch.cuda.synchronize()
    rc, rs = F.quantize_rows(to_bits(q_t), cfg.block)
    assert np.array_equal(q8.cpu().numpy(), rc)
    assert np.array_equal(qs.cpu().numpy(), rs)
    assert rs[0, 1, 3] == 0
    vc, vsr = F.quantize_v(to_bits(v_t), cfg.block)
    assert np.array_equal(v8_to_tokens(v8.cpu().numpy()), vc)
    assert np.array_equal(vs.cpu().numpy(), vsr)


def test_fused_reorder_quantization():
    """bsa_reorder_pool with E4M3 outputs and bsa_reorder_quantize_v: codes and scales
    bit-identical to the oracle's quantization of the reordered tensors; the other outputs
    unchanged (batch 2, ragged tail)."""
    cfgs = [Config("f8f", 4, 12, 21, 2, 128, 128, (4, 4, 8), 0.9, 2, 90 + i) for i in range(2)]
    qkv = [gen_qkv(c, gains=np.full(2, 1.5)) for c in cfgs]
    q = np.concatenate([x[0] for x in qkv], axis=0)
    v = np.concatenate([x[2] for x in qkv], axis=0)
    cfg = cfgs[0]
    grid = grid_of(cfg)
    B = cfg.block
    print(f"[gpu] fused fp8 reorder batch=2 N={cfg.N} n_blk={grid.n_blk}", flush=True)
    tq, tv = to_dev(q), to_dev(v)
    q_t, qbar, q8, qs = bsa.reorder_pool(tq, grid, fp8=True)
    none_t, qbar2, q8b, qsb = bsa.reorder_pool(tq, grid, tiled=False, fp8=True)
    v_t, v8, vs = bsa.reorder_quantize_v(tv, grid, tiled=True)
    _, v8b, vsb = bsa.reorder_quantize_v(tv, grid)
    plain_t, plain_bar = bsa.reorder_pool(tq, grid)
    torch.cuda.synchronize()
    assert none_t is None
    ref_q = O.reorder(q, cfg.T, cfg.H, cfg.W, cfg.tile, B)
    ref_v = O.reorder(v, cfg.T, cfg.H, cfg.W, cfg.tile, B)
    assert np.array_equal(to_bits(q_t), ref_q) and np.array_equal(to_bits(v_t), ref_v)
    assert torch.equal(qbar, plain_bar) and torch.equal(qbar2, plain_bar)
    rc, rs = F.quantize_rows(ref_q, B)
    for c8, sc in ((q8, qs), (q8b, qsb)):
        assert np.array_equal(c8.cpu().numpy(), rc)
        assert np.array_equal(sc.cpu().numpy(), rs)
    vc, vsr = F.quantize_v(ref_v, B)
    for c8, sc in ((v8, vs), (v8b, vsb)):
        assert np.array_equal(v8_to_tokens(c8.cpu().numpy()), vc)
        assert np.array_equal(sc.cpu().numpy(), vsr)


@pytest.mark.parametrize("expcast", [False, True], ids=["rne", "expcast"])
@pytest.mark.parametrize("grid3,heads,routed,seed,zero", [
    ((4, 12, 21), 3, True, 82, None),
    ((6, 24, 32), 1, False, 83, None),
    # Q and K of whole blocks zero (scale 0, so the softmax multiplier is floored): the last
    # block of head 1, which also holds the 16 pad keys of the ragged tail, and a middle block
    # of head 0; every row takes every block
    ((4, 12, 21), 2, False, 84, [(1, 7), (0, 3)])],
    ids=["routed", "split_full", "zero_blocks"])
def test_fp8_attention_within_bound(grid3, heads, routed, seed, zero, expcast):
    T, H, W = grid3
    cfg = Config("f8a", T, H, W, heads, 128, 128, (4, 4, 8), 0.9, 2, seed)
    grid, q_t, k_t, v_t = _tiled(cfg, zero_block=zero)
    n = grid.n_blk
    if routed:
        rp, ci, nnz = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor)
    else:                                         # every row full: long rows are split
        rp = torch.arange(0, heads * n + 1, dtype=torch.int32, device="cuda:0") * n
        ci = torch.arange(n, dtype=torch.int32, device="cuda:0").repeat(heads * n)
        nnz = rp[-1:]
    q8, qs = bsa.quantize_fp8(q_t, grid)
    k8, ks = bsa.quantize_fp8(k_t, grid)
    v8, vs = bsa.quantize_fp8(v_t, grid, v_layout=True)
    sc = attn_scale(128)
    out, lse = bsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8, vs, rp, ci, grid, sc, expcast=expcast)
    torch.cuda.synchronize()
    print(f"[gpu] fp8 attention {T}x{H}x{W} heads={heads} n_blk={n} nnz={int(nnz.item())} "
          f"expcast={expcast}", flush=True)
    _check_fp8(out, lse, q_t, k_t, v_t, rp, ci, nnz, cfg, sc, expcast)


def _check_fp8(out, lse, q_t, k_t, v_t, rp, ci, nnz, cfg, sc, expcast):
    """Every row of every (batch, head) within the oracle's cast bound (ExpCast or exact cast)
    of the exact attention over the dequantized inputs; pad rows zero."""
    N, B = cfg.N, cfg.block
    nb, heads = q_t.shape[0], q_t.shape[1]
    n = -(-N // B)
    nz = int(nnz.item())
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:nz].cpu().numpy().astype(np.int64)
    qc, qsr = F.quantize_rows(to_bits(q_t), B)
    kc, ksr = F.quantize_rows(to_bits(k_t), B)
    vc, vsr = F.quantize_v(to_bits(v_t), B)
    qd, kd, vd = (F.dequantize_rows(qc, qsr, B), F.dequantize_rows(kc, ksr, B),
                  F.dequantize_v(vc, vsr))
    Oref, Lref = O.sparse_attn(qd, kd, vd, rp_h, ci_h, N, B, sc)
    rows = [(bi, hh, i) for bi in range(nb) for hh in range(heads) for i in range(n)]
    if expcast:
        bnd = F.expcast_error_bound(qd, kd, vd, rp_h, ci_h, N, B, sc, rows)
    else:
        bo = F.attn_error_bound(qd, kd, vd, rp_h, ci_h, N, B, sc, rows)
        bnd = {r: (bo[r], np.zeros(bo[r].shape[0])) for r in rows}
    wabs = F.abs_weighted_v(qd, kd, vd, rp_h, ci_h, N, B, sc, rows)
    got = bf16_f64(out)
    lse_h = lse.cpu().numpy().astype(np.float64)
    worst = 0.0
    for (bi, hh, i) in rows:
        lo, hi = i * B, min((i + 1) * B, N)
        ref = Oref[bi, hh, lo:hi]
        tol = fp8_out_tol(bnd[(bi, hh, i)][0], ref, wabs[(bi, hh, i)])
        err = np.abs(got[bi, hh, lo:hi] - ref)
        assert np.all(err <= tol), (bi, hh, i, float((err / tol).max()))
        worst = max(worst, float((err / tol).max()))
        dl = np.abs(lse_h[bi, hh, lo:hi] - Lref[bi, hh, lo:hi])
        assert np.all(dl <= bnd[(bi, hh, i)][1] + 1e-3), (bi, hh, i, float(dl.max()))
    assert np.all(got[:, :, N:] == 0)
    # accuracy against the exact attention on the bf16 inputs (reported, not a bar)
    O16, _ = O.sparse_attn(to_bits(q_t), to_bits(k_t), to_bits(v_t), rp_h, ci_h, N, B, sc)
    d16 = np.abs(got[:, :, :N] - O16[:, :, :N])
    print(f"[gpu]   worst err/bound {worst:.3f}; vs bf16-input attention max-abs "
          f"{d16.max():.3e} mean-abs {d16.mean():.3e}", flush=True)


@pytest.mark.parametrize("expcast", [False, True], ids=["rne", "expcast"])
def test_fp8_attention_batch2(expcast):
    """Batch 2 (two differently seeded fields, two heads each, ragged tail), routed by
    bsa_score_and_route: every row of both batch entries within the cast bound."""
    cfgs = [Config("f8b", 4, 12, 21, 2, 128, 128, (4, 4, 8), 0.9, 2, 95 + i) for i in range(2)]
    qkv = [gen_qkv(c, gains=np.full(2, 1.5)) for c in cfgs]
    cfg = cfgs[0]
    grid = grid_of(cfg)
    q_t, k_t, v_t = (bsa.reorder(to_dev(np.concatenate([x[j] for x in qkv], axis=0)), grid)
                     for j in range(3))
    rp, ci, nnz = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor)
    q8, qs = bsa.quantize_fp8(q_t, grid)
    k8, ks = bsa.quantize_fp8(k_t, grid)
    v8, vs = bsa.quantize_fp8(v_t, grid, v_layout=True)
    sc = attn_scale(128)
    out, lse = bsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8, vs, rp, ci, grid, sc, expcast=expcast)
    torch.cuda.synchronize()
    print(f"[gpu] fp8 attention batch=2 heads=2 N={cfg.N} nnz={int(nnz.item())} "
          f"expcast={expcast}", flush=True)
    _check_fp8(out, lse, q_t, k_t, v_t, rp, ci, nnz, cfg, sc, expcast)
