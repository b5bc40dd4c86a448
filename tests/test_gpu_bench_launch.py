"""GPU parity of the layer step exactly as `bench.py` launches it, at the full sizes of the
video layers: every head in one launch, the caller-owned buffers and workspaces, the fused
reorder + block means, the routing from the means, the attention and the inverse reorder.

* bf16 on HunyuanVideo (the bench's default layer), Wan-480p and Wan-720p (all 24 / 40 / 40
  heads) and on Wan-480p under the Hilbert order: reorders bit-exact both ways, block means
  exact, masks accepted on every row, attention output within max-abs 2e-2 / mean-abs 2e-3 and
  LSE within 1e-3 on sampled rows.
* FP8 with the ExpCast cast on Wan-480p (the step of `bench.py --fp8 --expcast`): E4M3 codes
  and scales bit-exact on sampled heads, masks on every row, outputs and LSE within the
  oracle's ExpCast bounds on sampled rows."""
import ctypes
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from oracle import fp8 as F
from workloads import CONFIGS, gen_qkv

from fp8_support import fp8_out_tol, v8_to_tokens
from gpu_common import bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS, LSE_ABS = 2e-2, 2e-3, 1e-3


def _buffers(h, D, grid, dev):
    Np, n = grid.Npad, grid.n_blk
    rows = h * n
    return dict(
        q_t=torch.empty((1, h, Np, D), dtype=torch.bfloat16, device=dev),
        k_t=torch.empty((1, h, Np, D), dtype=torch.bfloat16, device=dev),
        v_t=torch.empty((1, h, Np, D), dtype=torch.bfloat16, device=dev),
        out_t=torch.empty((1, h, Np, D), dtype=torch.bfloat16, device=dev),
        out=torch.empty((1, grid.N, h, D), dtype=torch.bfloat16, device=dev),
        lse=torch.empty((1, h, Np), dtype=torch.float32, device=dev),
        row_ptr=torch.empty(rows + 1, dtype=torch.int32, device=dev),
        col_idx=torch.empty(rows * n, dtype=torch.int32, device=dev),
        nnz=torch.empty(1, dtype=torch.int32, device=dev),
        qbar=torch.empty((1, h, n, D), dtype=torch.float64, device=dev),
        kbar=torch.empty((1, h, n, D), dtype=torch.float64, device=dev),
        ws_r=torch.empty(bsa.route_workspace_bytes(1, h, D, grid), dtype=torch.uint8,
                         device=dev))


def _csr(b):
    nz = int(b["nnz"].item())
    rp = b["row_ptr"].cpu().numpy().astype(np.int64)
    ci = b["col_idx"][:nz].cpu().numpy().astype(np.int64)
    assert nz == rp[-1]
    return rp, ci


def _sub_csr(rp, ci, heads, n):
    """The CSR rows of the listed heads, renumbered as heads 0, 1, ..."""
    counts, cols = [], []
    for hh in heads:
        for i in range(n):
            r = hh * n + i
            counts.append(rp[r + 1] - rp[r])
            cols.append(ci[rp[r]:rp[r + 1]])
    return np.concatenate([[0], np.cumsum(counts)]), np.concatenate(cols)


def _routing_checks(cfg, grid, b, qt_ref, kt_ref):
    N, B, D = cfg.N, cfg.block, cfg.head_dim
    n = grid.n_blk
    qf, kf = O.widen_bf16(qt_ref), O.widen_bf16(kt_ref)
    assert np.array_equal(b["qbar"].cpu().numpy(), O.pool(qf, N, B))
    assert np.array_equal(b["kbar"].cpu().numpy(), O.pool(kf, N, B))
    ref = O.route(qf, kf, N, B, cfg.top_p, cfg.k_floor, 1.0 / math.sqrt(D))
    rp, ci = _csr(b)
    rep = O.check_mask(ref, rp, ci, cfg.top_p, cfg.k_floor)
    rows = qt_ref.shape[1] * n
    print(f"[gpu]   mask rows {rep.rows}: exact {rep.exact} tie {rep.tie} count {rep.count} "
          f"nnz {rp[-1]} sparsity {1 - rp[-1] / (rows * n):.4f}", flush=True)
    assert rep.rows == rows and rep.ok, rep.failures[:5]
    return rp, ci


@pytest.mark.parametrize("name,order", [("hunyuan720p", "tile"), ("wan480p", "tile"),
                                        ("wan720p", "tile"), ("wan480p", "hilbert")])
def test_bench_step_bf16(name, order):
    cfg = CONFIGS[name]
    dev = torch.device("cuda:0")
    D, B, N = cfg.head_dim, cfg.block, cfg.N
    print(f"[gpu] bench step {name} order={order}: all {cfg.heads} heads", flush=True)
    q, k, v = gen_qkv(cfg)
    h = q.shape[2]
    grid = grid_of(cfg)
    pi = None
    if order == "hilbert":
        grid = grid.with_order(bsa.hilbert_order(grid, device=dev))
        pi = O.hilbert_perm(cfg.T, cfg.H, cfg.W)
    b = _buffers(h, D, grid, dev)
    ws_a = torch.empty(bsa.attn_workspace_bytes(1, h, D, grid), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    qr, kr, vr = to_dev(q), to_dev(k), to_dev(v)
    bsa.reorder_pool(qr, grid, out=b["q_t"], pooled=b["qbar"])
    bsa.reorder_pool(kr, grid, out=b["k_t"], pooled=b["kbar"])
    bsa.reorder(vr, grid, out=b["v_t"])
    bsa.route_pooled(b["qbar"], b["kbar"], grid, cfg.top_p, cfg.k_floor, scale,
                     workspace=b["ws_r"], row_ptr=b["row_ptr"], col_idx=b["col_idx"],
                     nnz=b["nnz"])
    bsa.sparse_attn_fwd(b["q_t"], b["k_t"], b["v_t"], b["row_ptr"], b["col_idx"], grid, scale,
                        out=b["out_t"], lse=b["lse"], workspace=ws_a)
    bsa.reorder(b["out_t"], grid, inverse=True, out=b["out"])
    torch.cuda.synchronize()
    refs = [O.reorder(x, cfg.T, cfg.H, cfg.W, cfg.tile, B, pi=pi) for x in (q, k, v)]
    for t, ref in zip(("q_t", "k_t", "v_t"), refs):
        assert np.array_equal(to_bits(b[t]), ref), t
    rp, ci = _routing_checks(cfg, grid, b, refs[0], refs[1])
    heads = [0, h // 2, h - 1]
    qblocks = list(range(0, grid.n_blk, 16)) + [grid.n_blk - 1]
    sc = float(np.float32(scale))
    Oref, Lref = O.sparse_attn(refs[0], refs[1], refs[2], rp, ci, N, B, sc, heads=heads,
                               qblocks=qblocks)
    got, lse = bf16_f64(b["out_t"]), b["lse"].cpu().numpy().astype(np.float64)
    errs = []
    for hh in heads:
        for i in qblocks:
            lo, hi = i * B, min((i + 1) * B, N)
            errs.append(np.abs(got[0, hh, lo:hi] - Oref[0, hh, lo:hi]))
            assert np.abs(lse[0, hh, lo:hi] - Lref[0, hh, lo:hi]).max() <= LSE_ABS, (hh, i)
    d = np.concatenate([e.ravel() for e in errs])
    print(f"[gpu]   {len(heads)} heads x {len(qblocks)} query blocks: out max-abs "
          f"{d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= MAX_ABS and d.mean() <= MEAN_ABS
    assert np.all(got[:, :, N:] == 0)
    assert np.array_equal(to_bits(b["out"]),
                          O.inverse_reorder(to_bits(b["out_t"]), cfg.T, cfg.H, cfg.W, cfg.tile,
                                            pi=pi))


def test_bench_step_fp8_expcast():
    cfg = CONFIGS["wan480p"]
    dev = torch.device("cuda:0")
    D, B, N = cfg.head_dim, cfg.block, cfg.N
    print(f"[gpu] bench step wan480p fp8 expcast: all {cfg.heads} heads", flush=True)
    q, k, v = gen_qkv(cfg)
    h = q.shape[2]
    grid = grid_of(cfg)
    n = grid.n_blk
    b = _buffers(h, D, grid, dev)
    q8 = torch.empty((1, h, grid.Npad, D), dtype=torch.uint8, device=dev)
    k8 = torch.empty_like(q8)
    v8 = torch.empty((1, h, n, D, B), dtype=torch.uint8, device=dev)
    qs = torch.empty((1, h, n), dtype=torch.float32, device=dev)
    ks = torch.empty_like(qs)
    vs = torch.empty((1, h), dtype=torch.float32, device=dev)
    g, shp = grid._c(), bsa._shape(1, h, D)
    ws_bytes = int(bsa.lib().bsa_attn_fp8_workspace_bytes(ctypes.byref(shp), ctypes.byref(g)))
    ws_a = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(D)
    qr, kr, vr = to_dev(q), to_dev(k), to_dev(v)
    bsa.reorder_pool(qr, grid, tiled=False, pooled=b["qbar"], fp8=True, x8=q8, x8_scales=qs)
    bsa.reorder_pool(kr, grid, tiled=False, pooled=b["kbar"], fp8=True, x8=k8, x8_scales=ks)
    bsa.reorder_quantize_v(vr, grid, v8=v8, v_scales=vs)
    bsa.route_pooled(b["qbar"], b["kbar"], grid, cfg.top_p, cfg.k_floor, scale,
                     workspace=b["ws_r"], row_ptr=b["row_ptr"], col_idx=b["col_idx"],
                     nnz=b["nnz"])
    sc = float(np.float32(scale))
    bsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8, vs, b["row_ptr"], b["col_idx"], grid, sc,
                            out=b["out_t"], lse=b["lse"], workspace=ws_a, expcast=True)
    bsa.reorder(b["out_t"], grid, inverse=True, out=b["out"])
    torch.cuda.synchronize()
    refs = [O.reorder(x, cfg.T, cfg.H, cfg.W, cfg.tile, B) for x in (q, k, v)]
    rp, ci = _routing_checks(cfg, grid, b, refs[0], refs[1])
    heads = [0, h - 1]
    qc, qsr = F.quantize_rows(refs[0][:, heads], B)
    kc, ksr = F.quantize_rows(refs[1][:, heads], B)
    vc, vsr = F.quantize_v(refs[2][:, heads], B)
    for got8, want in ((q8[:, heads], qc), (qs[:, heads], qsr), (k8[:, heads], kc),
                       (ks[:, heads], ksr), (vs[:, heads], vsr)):
        assert np.array_equal(got8.cpu().numpy(), want)
    assert np.array_equal(v8_to_tokens(v8[:, heads].cpu().numpy()), vc)
    qd, kd, vd = (F.dequantize_rows(qc, qsr, B), F.dequantize_rows(kc, ksr, B),
                  F.dequantize_v(vc, vsr))
    srp, sci = _sub_csr(rp, ci, heads, n)
    qblocks = list(range(0, n, 16)) + [n - 1]
    Oref, Lref = O.sparse_attn(qd, kd, vd, srp, sci, N, B, sc, qblocks=qblocks)
    rows = [(0, j, i) for j in range(len(heads)) for i in qblocks]
    bnd = F.expcast_error_bound(qd, kd, vd, srp, sci, N, B, sc, rows)
    wabs = F.abs_weighted_v(qd, kd, vd, srp, sci, N, B, sc, rows)
    got, lse = bf16_f64(b["out_t"]), b["lse"].cpu().numpy().astype(np.float64)
    worst = 0.0
    for (_, j, i) in rows:
        hh = heads[j]
        lo, hi = i * B, min((i + 1) * B, N)
        ref = Oref[0, j, lo:hi]
        tol = fp8_out_tol(bnd[(0, j, i)][0], ref, wabs[(0, j, i)])
        err = np.abs(got[0, hh, lo:hi] - ref)
        assert np.all(err <= tol), (hh, i, float((err / tol).max()))
        worst = max(worst, float((err / tol).max()))
        dl = np.abs(lse[0, hh, lo:hi] - Lref[0, j, lo:hi])
        assert np.all(dl <= bnd[(0, j, i)][1] + 1e-3), (hh, i, float(dl.max()))
    print(f"[gpu]   {len(rows)} sampled rows: worst err/bound {worst:.3f}", flush=True)
    assert np.all(got[:, :, N:] == 0)
    assert np.array_equal(to_bits(b["out"]),
                          O.inverse_reorder(to_bits(b["out_t"]), cfg.T, cfg.H, cfg.W, cfg.tile))
