"""GPU test of bsa_sparse_attn_fwd_noalloc, the attention entry point that allocates nothing
(its schedule and split-row partials live in the library's static per-device scratch): called
raw through the C ABI twice in a row, the second time on a smaller input, each output and LSE
bit-identical to bsa_sparse_attn_fwd's on the same inputs (and therefore inside the parity
bars: max-abs 2e-2, mean-abs 2e-3, LSE 1e-3 against the oracle, checked too)."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv

from gpu_common import attn_scale, bf16_f64, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _inputs(cfg, dense):
    q, k, v = gen_qkv(cfg, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in (q, k, v))
    n, h = grid.n_blk, cfg.heads
    if dense:                                  # every row keeps every block: rows are split
        rp = torch.arange(0, h * n + 1, dtype=torch.int32, device="cuda:0") * n
        ci = torch.arange(n, dtype=torch.int32, device="cuda:0").repeat(h * n)
    else:
        rp, ci, _ = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor)
    return grid, q_t, k_t, v_t, rp, ci


def _noalloc(grid, q_t, k_t, v_t, rp, ci, scale):
    b, h, Np, D = q_t.shape
    out = torch.full_like(q_t, float("nan"))
    lse = torch.full((b, h, Np), float("nan"), dtype=torch.float32, device=q_t.device)
    g, s = grid._c(), bsa._shape(b, h, D)
    L = bsa.lib()
    st = L.bsa_sparse_attn_fwd_noalloc(
        q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(), rp.data_ptr(), ci.data_ptr(),
        ctypes.byref(s), ctypes.byref(g), ctypes.c_float(scale), out.data_ptr(),
        lse.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.bsa_last_error()
    return out, lse


def test_noalloc_matches_workspace_entry_point_twice():
    cases = [(Config("na_big", 6, 24, 32, 2, 128, 128, (4, 4, 8), 0.9, 2, 141), True),
             (Config("na_small", 2, 16, 16, 2, 64, 64, (4, 4, 4), 0.9, 2, 142), False)]
    for cfg, dense in cases:
        grid, q_t, k_t, v_t, rp, ci = _inputs(cfg, dense)
        sc = attn_scale(cfg.head_dim)
        print(f"[gpu] noalloc {cfg.name}: {cfg.T}x{cfg.H}x{cfg.W} heads={cfg.heads} "
              f"D={cfg.head_dim} B={cfg.block} dense={dense}", flush=True)
        ref_out, ref_lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, sc)
        out, lse = _noalloc(grid, q_t, k_t, v_t, rp, ci, sc)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        # the parity bars against the oracle on the same CSR
        N, B = cfg.N, cfg.block
        nz = int(rp[-1].item())
        Oref, Lref = O.sparse_attn(to_bits(q_t), to_bits(k_t), to_bits(v_t),
                                   rp.cpu().numpy().astype(np.int64),
                                   ci[:nz].cpu().numpy().astype(np.int64), N, B, sc)
        d = np.abs(bf16_f64(out)[:, :, :N] - Oref[:, :, :N])
        dl = np.abs(lse.cpu().numpy().astype(np.float64)[:, :, :N] - Lref[:, :, :N])
        print(f"[gpu]   bit-identical; vs oracle max-abs {d.max():.2e} mean-abs "
              f"{d.mean():.2e} lse {dl.max():.2e}", flush=True)
        assert d.max() <= 2e-2 and d.mean() <= 2e-3 and dl.max() <= 1e-3


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """A workspace need above the static scratch is refused on the host (nothing launched)."""
    L = bsa.lib()
    g = bsa.Grid(64, 128, 128, (4, 4, 8), 128)._c()            # n_blk 8192 > 4096: unsupported
    s = bsa._shape(1, 1, 128)
    fake = 1 << 20
    st = L.bsa_sparse_attn_fwd_noalloc(fake, fake, fake, fake, fake, ctypes.byref(s),
                                       ctypes.byref(g), ctypes.c_float(0.1), fake, None, None)
    assert st != 0
    g2 = bsa.Grid(33, 45, 80, (4, 4, 8), 128)._c()             # 929 blocks a row
    s2 = bsa._shape(1, 512, 128)                              # 475,648 rows
    st = L.bsa_sparse_attn_fwd_noalloc(fake, fake, fake, fake, fake, ctypes.byref(s2),
                                       ctypes.byref(g2), ctypes.c_float(0.1), fake, None, None)
    assert st == -3 and b"static scratch" in L.bsa_last_error()
