"""GPU tests at the largest sizes the attention and routing accept, through the C ABI.

* 4096 key blocks a row (the planner's limit), D = B = 64: the routed CSR of a whole 64^3
  latent grid (one head) accepted row by row against the fp64 oracle's routing, and the
  attention over it against the oracle on sampled rows (first, last, longest).
* 4096 key blocks a row, D = B = 128 (N = 524,288): a caller CSR where every row keeps its
  first, own and last block and two rows keep all 4096, so those rows are split into many
  chunks and merged; the oracle checks the dense rows, the edge rows and the last row index
  (4095, the top of the planner's 12-bit row field).
* 2048 batch x heads (the planner's head limit): routing and attention over 2048 heads of a
  tiny grid, every mask row checked and sampled heads' outputs against the oracle.
* The FP8 kernel on the same 4096-block CSR, both probability casts, against the oracle's
  derived bounds.
* One past each limit (4097 blocks, 2049 heads) is refused on the host before any launch.
Bars as everywhere: output max-abs 2e-2 and mean-abs 2e-3, LSE 1e-3, masks per R15.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, bf16_bits_from_f64, gen_qkv

from gpu_common import attn_scale, bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _check_rows(q_t, k_t, v_t, rp, ci, out_t, lse, N, B, sc, rows, heads=1):
    """Oracle attention on the listed (head, query block) rows of the GPU's own CSR."""
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy().astype(np.int64)
    got = bf16_f64(out_t)
    lse_h = lse.cpu().numpy().astype(np.float64)
    qb, kb, vb = to_bits(q_t), to_bits(k_t), to_bits(v_t)
    worst = 0.0
    for hh in sorted({h for h, _ in rows}):
        blocks = sorted({i for h, i in rows if h == hh})
        Oref, Lref = O.sparse_attn(qb, kb, vb, rp_h, ci_h, N, B, sc, heads=[hh], qblocks=blocks)
        for i in blocks:
            lo, hi = i * B, min((i + 1) * B, N)
            d = np.abs(got[0, hh, lo:hi] - Oref[0, hh, lo:hi])
            dl = np.abs(lse_h[0, hh, lo:hi] - Lref[0, hh, lo:hi])
            assert d.max() <= 2e-2 and d.mean() <= 2e-3, (hh, i, d.max(), d.mean())
            assert dl.max() <= 1e-3, (hh, i, dl.max())
            worst = max(worst, float(d.max()))
    return worst


def test_route_and_attention_4096_blocks():
    cfg = Config("lim4096", 64, 64, 64, 1, 64, 64, (4, 4, 4), 0.9, 4, 61)
    q, k, v = gen_qkv(cfg, gains=np.full(1, 1.5))
    grid = grid_of(cfg)
    n, N, B = grid.n_blk, cfg.N, cfg.block
    assert n == 4096
    print(f"[gpu] limits: route + attention, N={N} n_blk={n}", flush=True)
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in (q, k, v))
    scale = 1.0 / math.sqrt(cfg.head_dim)
    rp, ci, nnz = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor, scale)[:3]
    sc = attn_scale(cfg.head_dim)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, sc)
    torch.cuda.synchronize()
    nz = int(nnz.item())
    ref = O.route(to_bits(q_t), to_bits(k_t), N, B, cfg.top_p, cfg.k_floor, scale)
    rep = O.check_mask(ref, rp.cpu().numpy(), ci[:nz].cpu().numpy(), cfg.top_p, cfg.k_floor)
    print(f"[gpu]   mask rows {rep.rows}: exact {rep.exact} tie {rep.tie} count {rep.count} "
          f"nnz {nz}", flush=True)
    assert rep.ok, rep.failures[:5]
    counts = np.diff(rp.cpu().numpy())
    rows = [(0, 0), (0, n - 1), (0, int(np.argmax(counts))), (0, n // 2)]
    worst = _check_rows(q_t, k_t, v_t, rp, ci, out_t, lse, N, B, sc, rows)
    print(f"[gpu]   attention rows {rows}: worst max-abs {worst:.3e}", flush=True)


def test_attention_4096_blocks_split_rows():
    B = D = 128
    n = 4096
    N = n * B - 45                                     # ragged last block
    grid = bsa.Grid(1, 1, N, (1, 1, B), B)
    assert grid.n_blk == n
    rng = np.random.default_rng(63)
    print(f"[gpu] limits: attention D=B=128, N={N} n_blk={n}, dense rows 2048 and 4095",
          flush=True)
    tens = []
    for _ in range(3):
        t = np.zeros((1, 1, grid.Npad, D))
        t[0, 0, :N] = rng.standard_normal((N, D))
        tens.append(torch.from_numpy(bf16_bits_from_f64(t).view(np.int16)).view(
            torch.bfloat16).to("cuda:0"))
    q_t, k_t, v_t = tens
    rows = []
    for i in range(n):
        cols = np.arange(n) if i in (n // 2, n - 1) else np.unique([0, i, n - 1])
        rows.append(cols)
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ci = np.concatenate(rows).astype(np.int32)
    rp_d, ci_d = torch.from_numpy(rp).to("cuda:0"), torch.from_numpy(ci).to("cuda:0")
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp_d, ci_d, grid, sc)
    torch.cuda.synchronize()
    assert np.all(bf16_f64(out_t)[:, :, N:] == 0)
    check = [(0, 0), (0, 1), (0, n // 2), (0, n - 2), (0, n - 1)]
    worst = _check_rows(q_t, k_t, v_t, rp_d, ci_d, out_t, lse, N, B, sc, check)
    print(f"[gpu]   rows {check}: worst max-abs {worst:.3e}", flush=True)


def test_attention_2048_heads():
    heads = 2048
    cfg = Config("lim_heads", 2, 4, 16, heads, 64, 64, (2, 4, 8), 0.9, 1, 62)
    grid = grid_of(cfg)
    N, B, D = cfg.N, cfg.block, cfg.head_dim
    rng = np.random.default_rng(64)
    print(f"[gpu] limits: {heads} heads, N={N} n_blk={grid.n_blk}", flush=True)
    raw = [bf16_bits_from_f64(rng.standard_normal((1, N, heads, D)) * g)
           for g in (1.5, 1.0, 1.0)]
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in raw)
    scale = 1.0 / math.sqrt(D)
    rp, ci, nnz = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor, scale)[:3]
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, sc)
    torch.cuda.synchronize()
    nz = int(nnz.item())
    ref = O.route(to_bits(q_t), to_bits(k_t), N, B, cfg.top_p, cfg.k_floor, scale)
    rep = O.check_mask(ref, rp.cpu().numpy(), ci[:nz].cpu().numpy(), cfg.top_p, cfg.k_floor)
    print(f"[gpu]   mask rows {rep.rows}: exact {rep.exact} tie {rep.tie} nnz {nz}", flush=True)
    assert rep.ok, rep.failures[:5]
    check = [(h, i) for h in (0, 1, 1023, 2047) for i in range(grid.n_blk)]
    worst = _check_rows(q_t, k_t, v_t, rp, ci, out_t, lse, N, B, sc, check)
    print(f"[gpu]   heads 0, 1, 1023, 2047: worst max-abs {worst:.3e}", flush=True)


def test_one_past_each_limit_is_refused():
    dev = "cuda:0"
    # 2049 heads of a one-block grid
    g = bsa.Grid(1, 1, 64, (1, 1, 64), 64)
    x = torch.zeros((1, 2049, g.Npad, 64), dtype=torch.bfloat16, device=dev)
    rp = torch.arange(0, 2049 * g.n_blk + 1, dtype=torch.int32, device=dev)
    ci = torch.zeros(2049 * g.n_blk, dtype=torch.int32, device=dev)
    with pytest.raises(bsa.BsaError, match="exceeds"):
        bsa.sparse_attn_fwd(x, x, x, rp, ci, g, 0.125)
    # 4097 key blocks a row
    g = bsa.Grid(1, 1, 4097 * 64, (1, 1, 64), 64)
    assert g.n_blk == 4097
    x = torch.zeros((1, 1, g.Npad, 64), dtype=torch.bfloat16, device=dev)
    rp = torch.arange(0, g.n_blk + 1, dtype=torch.int32, device=dev)
    ci = torch.zeros(g.n_blk, dtype=torch.int32, device=dev)
    with pytest.raises(bsa.BsaError, match="exceeds"):
        bsa.sparse_attn_fwd(x, x, x, rp, ci, g, 0.125)


@pytest.mark.parametrize("expcast", [False, True], ids=["rne", "expcast"])
def test_fp8_attention_4096_blocks_split_rows(expcast):
    """The FP8 kernel at 4096 key blocks a row with the same CSR as above (dense rows split into
    about 200 chunks and merged): outputs within the oracle's cast bound plus the fp32 and bf16
    terms (tests/fp8_support.fp8_out_tol), LSE within 1e-3 (plus the ExpCast bound)."""
    from oracle import fp8 as F
    from fp8_support import fp8_out_tol
    B = D = 128
    n = 4096
    N = n * B - 45
    grid = bsa.Grid(1, 1, N, (1, 1, B), B)
    rng = np.random.default_rng(65)
    print(f"[gpu] limits: fp8 attention expcast={expcast} N={N} n_blk={n}", flush=True)
    tens = []
    for _ in range(3):
        t = np.zeros((1, 1, grid.Npad, D))
        t[0, 0, :N] = rng.standard_normal((N, D))
        tens.append(torch.from_numpy(bf16_bits_from_f64(t).view(np.int16)).view(
            torch.bfloat16).to("cuda:0"))
    q_t, k_t, v_t = tens
    rows = [np.arange(n) if i in (n // 2, n - 1) else np.unique([0, i, n - 1]) for i in range(n)]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    ci = np.concatenate(rows).astype(np.int64)
    rp_d = torch.from_numpy(rp.astype(np.int32)).to("cuda:0")
    ci_d = torch.from_numpy(ci.astype(np.int32)).to("cuda:0")
    q8, qs = bsa.quantize_fp8(q_t, grid)
    k8, ks = bsa.quantize_fp8(k_t, grid)
    v8, vs = bsa.quantize_fp8(v_t, grid, v_layout=True)
    sc = attn_scale(D)
    out, lse = bsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8, vs, rp_d, ci_d, grid, sc,
                                       expcast=expcast)
    torch.cuda.synchronize()
    qc, qsr = F.quantize_rows(to_bits(q_t), B)
    kc, ksr = F.quantize_rows(to_bits(k_t), B)
    vc, vsr = F.quantize_v(to_bits(v_t), B)
    qd, kd, vd = (F.dequantize_rows(qc, qsr, B), F.dequantize_rows(kc, ksr, B),
                  F.dequantize_v(vc, vsr))
    check = [(0, 0, i) for i in (0, 1, n // 2, n - 2, n - 1)]
    if expcast:
        bnd = F.expcast_error_bound(qd, kd, vd, rp, ci, N, B, sc, check)
    else:
        bo = F.attn_error_bound(qd, kd, vd, rp, ci, N, B, sc, check)
        bnd = {r: (bo[r], np.zeros(bo[r].shape[0])) for r in check}
    wabs = F.abs_weighted_v(qd, kd, vd, rp, ci, N, B, sc, check)
    Oref, Lref = O.sparse_attn(qd, kd, vd, rp, ci, N, B, sc, heads=[0],
                               qblocks=[i for _, _, i in check])
    got = bf16_f64(out)
    lse_h = lse.cpu().numpy().astype(np.float64)
    worst = 0.0
    for r in check:
        i = r[2]
        lo, hi = i * B, min((i + 1) * B, N)
        ref = Oref[0, 0, lo:hi]
        tol = fp8_out_tol(bnd[r][0], ref, wabs[r])
        err = np.abs(got[0, 0, lo:hi] - ref)
        assert np.all(err <= tol), (i, float((err / tol).max()))
        worst = max(worst, float((err / tol).max()))
        dl = np.abs(lse_h[0, 0, lo:hi] - Lref[0, 0, lo:hi])
        assert np.all(dl <= bnd[r][1] + 1e-3), (i, float(dl.max()))
    assert np.all(got[:, :, N:] == 0)
    print(f"[gpu]   rows {[i for _, _, i in check]}: worst err/bound {worst:.3f}", flush=True)
