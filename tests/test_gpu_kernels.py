"""GPU tests of each call on its own, through the C ABI binding.

* Guard regions: every output (and the workspaces) sits inside a larger buffer filled with a
  canary pattern; after the calls the canary bytes must be untouched and the results equal to a
  run into plain buffers.
* Attention on caller-supplied CSRs (not produced by the router): random masks with mixed row
  densities, full rows, single-block rows and a ragged last block, against the fp64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv

from gpu_common import attn_scale, bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of canary before and after every output
CANARY = 0xA5


def guarded(nbytes, dtype, shape):
    """A tensor of `shape` inside a canary-filled uint8 buffer; returns (view, buffer)."""
    buf = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda:0")
    view = buf[GUARD:GUARD + nbytes].view(dtype).view(shape)
    return view, buf


def intact(buf):
    b = buf.cpu().numpy()
    return bool(np.all(b[:GUARD] == CANARY) and np.all(b[-GUARD:] == CANARY))


CFG = Config("guard", 3, 10, 13, 3, 128, 128, (2, 4, 4), 0.85, 2, 21)   # ragged tail, D=B=128


def test_guard_regions_untouched():
    cfg = CFG
    q, k, v = gen_qkv(cfg, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    h, D, n = cfg.heads, cfg.head_dim, grid.n_blk
    rows = h * n
    print(f"[gpu] guard: N={cfg.N} n_blk={n} heads={h} D={D}", flush=True)
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    tshape = (1, h, grid.Npad, D)
    tbytes = int(np.prod(tshape)) * 2
    q_t, gq = guarded(tbytes, torch.bfloat16, tshape)
    k_t, gk = guarded(tbytes, torch.bfloat16, tshape)
    v_t, gv = guarded(tbytes, torch.bfloat16, tshape)
    bsa.reorder(tq, grid, out=q_t)
    bsa.reorder(tk, grid, out=k_t)
    bsa.reorder(tv, grid, out=v_t)
    row_ptr, g1 = guarded(4 * (rows + 1), torch.int32, (rows + 1,))
    col_idx, g2 = guarded(4 * rows * n, torch.int32, (rows * n,))
    nnz, g3 = guarded(4, torch.int32, (1,))
    scores, g4 = guarded(8 * h * n * n, torch.float64, (1, h, n, n))
    wsr_n = bsa.route_workspace_bytes(1, h, D, grid)
    ws_r, g5 = guarded(wsr_n, torch.uint8, (wsr_n,))
    scale = 1.0 / math.sqrt(D)
    lib, s = bsa.lib(), bsa._shape(1, h, D)
    import ctypes
    st = lib.bsa_score_and_route(q_t.data_ptr(), k_t.data_ptr(), ctypes.byref(s),
                                 ctypes.byref(grid._c()), float(cfg.top_p), int(cfg.k_floor),
                                 scale, row_ptr.data_ptr(), col_idx.data_ptr(), nnz.data_ptr(),
                                 scores.data_ptr(), ws_r.data_ptr(), wsr_n,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0
    out_t, g6 = guarded(tbytes, torch.bfloat16, tshape)
    lse, g7 = guarded(4 * h * grid.Npad, torch.float32, (1, h, grid.Npad))
    wsa_n = bsa.attn_workspace_bytes(1, h, D, grid)
    ws_a, g8 = guarded(wsa_n, torch.uint8, (wsa_n,))
    bsa.sparse_attn_fwd(q_t, k_t, v_t, row_ptr, col_idx, grid, attn_scale(D), out=out_t,
                        lse=lse, workspace=ws_a)
    out, g9 = guarded(int(np.prod(q.shape)) * 2, torch.bfloat16, tuple(q.shape))
    bsa.reorder(out_t, grid, inverse=True, out=out)
    torch.cuda.synchronize()
    for name, g in (("q_t", gq), ("k_t", gk), ("v_t", gv), ("row_ptr", g1), ("col_idx", g2),
                    ("nnz", g3), ("scores", g4), ("route ws", g5), ("out_t", g6), ("lse", g7),
                    ("attn ws", g8), ("out", g9)):
        assert intact(g), f"guard bytes of {name} overwritten"
    # same results as the path into plain buffers
    from gpu_common import run_path
    ref = run_path(grid, q, k, v, cfg.top_p, cfg.k_floor)
    nz = int(nnz.item())
    assert nz == ref["nnz"]
    assert np.array_equal(row_ptr.cpu().numpy(), ref["row_ptr"])
    assert np.array_equal(col_idx[:nz].cpu().numpy(), ref["col_idx"])
    assert np.array_equal(to_bits(out_t), ref["out_bits"])
    assert np.array_equal(lse.cpu().numpy().astype(np.float64), ref["lse"])


def random_csr(rng, heads, n, kinds):
    """CSR over heads * n rows; kinds cycles per row: 'full', 'one', 'rand', 'empty'."""
    rp = [0]
    cols = []
    for r in range(heads * n):
        kind = kinds[r % len(kinds)]
        if kind == "empty":
            c = np.zeros(0, np.int64)
        elif kind == "full":
            c = np.arange(n)
        elif kind == "one":
            c = np.array([rng.integers(n)])
        else:
            m = int(rng.integers(1, n + 1))
            c = np.sort(rng.choice(n, size=m, replace=False))
        cols.extend(c.tolist())
        rp.append(len(cols))
    return np.asarray(rp, np.int64), np.asarray(cols, np.int64)


@pytest.mark.parametrize("D,B,heads,grid3,tile,kinds,seed", [
    (128, 128, 2, (4, 12, 21), (4, 4, 8), ["rand", "full", "one", "rand"], 31),
    (64, 64, 3, (3, 10, 13), (2, 4, 4), ["rand", "one", "full"], 32),
    (128, 64, 2, (4, 12, 20), (4, 4, 4), ["full", "rand"], 33),
    (64, 128, 2, (4, 12, 21), (4, 4, 8), ["one", "rand", "full"], 34),
    # one head, every row full: few long rows, so the planner splits and merges them
    (128, 128, 1, (6, 24, 32), (4, 4, 8), ["full"], 35),
], ids=["d128b128", "d64b64", "d128b64", "d64b128", "split_full"])
def test_attention_on_given_csr(D, B, heads, grid3, tile, kinds, seed):
    T, H, W = grid3
    cfg = Config("csr", T, H, W, heads, D, B, tile, 1.0, 1, seed)
    q, k, v = gen_qkv(cfg, gains=np.full(heads, 1.5))
    grid = grid_of(cfg)
    n, N = grid.n_blk, cfg.N
    rng = np.random.default_rng(seed)
    rp, ci = random_csr(rng, heads, n, kinds)
    print(f"[gpu] csr D={D} B={B} heads={heads} n_blk={n} nnz={len(ci)}", flush=True)
    q_t = bsa.reorder(to_dev(q), grid)
    k_t = bsa.reorder(to_dev(k), grid)
    v_t = bsa.reorder(to_dev(v), grid)
    rp_d = torch.from_numpy(rp.astype(np.int32)).to("cuda:0")
    ci_d = torch.from_numpy(ci.astype(np.int32)).to("cuda:0")
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp_d, ci_d, grid, sc)
    torch.cuda.synchronize()
    Oref, Lref = O.sparse_attn(to_bits(q_t), to_bits(k_t), to_bits(v_t), rp, ci, N, B, sc)
    got = bf16_f64(out_t)[:, :, :N]
    d = np.abs(got - Oref[:, :, :N])
    print(f"[gpu]   out max-abs {d.max():.3e} mean-abs {d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    dl = np.abs(lse.cpu().numpy().astype(np.float64)[:, :, :N] - Lref[:, :, :N])
    assert dl.max() <= 1e-3
    assert np.all(bf16_f64(out_t)[:, :, N:] == 0)


@pytest.mark.parametrize("D", [8, 64, 128, 136])
def test_reorder_batched_any_head_dim(D):
    """Both directions bit-exact for batch 3, a ragged grid with truncated tiles on every axis,
    and head sizes on the compile-time (64, 128) and runtime (8, 136) paths."""
    T, H, W, tile, B, heads, batch = 3, 10, 13, (2, 4, 4), 64, 3, 3
    rng = np.random.default_rng(40 + D)
    N = T * H * W
    x = rng.integers(0, 1 << 16, size=(batch, N, heads, D), dtype=np.uint16)
    grid = bsa.Grid(T, H, W, tile, B)
    print(f"[gpu] reorder batch={batch} N={N} heads={heads} D={D}", flush=True)
    xt = bsa.reorder(to_dev(x), grid)
    ref = O.reorder(x, T, H, W, tile, B)
    assert np.array_equal(to_bits(xt), ref)
    back = bsa.reorder(xt, grid, inverse=True)
    assert np.array_equal(to_bits(back), x)


@pytest.mark.parametrize("D,B,fp8", [(128, 128, False), (64, 64, False), (128, 128, True)],
                         ids=["d128", "d64", "fp8"])
def test_attention_empty_rows(D, B, fp8):
    """Rows that keep no block (every 4th row and the last row of the layer) are written as
    zeros, output and LSE, like pad rows; the other rows match the oracle as usual."""
    cfg = Config("empty", 4, 12, 21, 2, D, B, (4, 4, 8) if B == 128 else (2, 4, 8), 1.0, 1, 36)
    q, k, v = gen_qkv(cfg, gains=np.full(2, 1.5))
    grid = grid_of(cfg)
    n, N = grid.n_blk, cfg.N
    rng = np.random.default_rng(37)
    rp, ci = random_csr(rng, 2, n, ["empty", "rand", "full", "one"])
    empty = [r for r in range(2 * n) if r % 4 == 0 or r == 2 * n - 1]
    keep = [np.sort(ci[rp[r]:rp[r + 1]]) if r not in empty else np.zeros(0, np.int64)
            for r in range(2 * n)]
    rp = np.concatenate([[0], np.cumsum([len(x) for x in keep])]).astype(np.int64)
    ci = np.concatenate(keep).astype(np.int64)
    print(f"[gpu] empty rows D={D} B={B} fp8={fp8} rows={2 * n} empty={len(empty)}", flush=True)
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in (q, k, v))
    rp_d = torch.from_numpy(rp.astype(np.int32)).to("cuda:0")
    ci_d = torch.from_numpy(ci.astype(np.int32)).to("cuda:0")
    sc = attn_scale(D)
    if fp8:
        q8, qs = bsa.quantize_fp8(q_t, grid)
        k8, ks = bsa.quantize_fp8(k_t, grid)
        v8, vs = bsa.quantize_fp8(v_t, grid, v_layout=True)
        out_t, lse = bsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8, vs, rp_d, ci_d, grid, sc)
    else:
        out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp_d, ci_d, grid, sc)
    torch.cuda.synchronize()
    got = bf16_f64(out_t)
    lse_h = lse.cpu().numpy().astype(np.float64)
    for r in empty:
        hh, i = divmod(r, n)
        assert np.all(got[0, hh, i * B:(i + 1) * B] == 0) and np.all(lse_h[0, hh, i * B:(i + 1) * B] == 0)
    assert np.all(got[:, :, N:] == 0)
    if fp8:
        # the non-empty rows against the FP8 bound are covered by test_gpu_fp8; here only
        # that they were computed (finite, not all zero)
        for r in range(2 * n):
            if r in empty:
                continue
            hh, i = divmod(r, n)
            blk = got[0, hh, i * B:min((i + 1) * B, N)]
            assert np.all(np.isfinite(blk)) and np.any(blk != 0)
        return
    for hh in range(2):
        blocks = [i for i in range(n) if hh * n + i not in empty]
        Oref, Lref = O.sparse_attn(to_bits(q_t), to_bits(k_t), to_bits(v_t), rp, ci, N, B, sc,
                                   heads=[hh], qblocks=blocks)
        for i in blocks:
            lo, hi = i * B, min((i + 1) * B, N)
            d = np.abs(got[0, hh, lo:hi] - Oref[0, hh, lo:hi])
            assert d.max() <= 2e-2, (hh, i, d.max())
            assert np.abs(lse_h[0, hh, lo:hi] - Lref[0, hh, lo:hi]).max() <= 1e-3
