"""GPU test of mask reuse across denoising steps (MaskReuse / layer(mask=...)) through the C
ABI: on drifting inputs, routed steps produce masks the oracle accepts for their own inputs,
reused steps run the attention of their own inputs over the earlier step's CSR, and both match
the oracle's attention on that CSR within the bf16 bars."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv_steps

from gpu_common import attn_scale, grid_of, to_bits, to_dev

pytestmark = pytest.mark.gpu


def test_mask_reuse_over_drifting_steps():
    cfg = Config("reuse", 4, 12, 21, 3, 128, 128, (4, 4, 8), 0.9, 2, 103)
    T, H, W, B, D, N = cfg.T, cfg.H, cfg.W, cfg.block, cfg.head_dim, cfg.N
    steps = gen_qkv_steps(cfg, [0, 1, 2], drift=0.4, gains=np.full(cfg.heads, 1.5))
    grid = grid_of(cfg)
    reuse = bsa.MaskReuse(2)
    scale, sc = 1.0 / math.sqrt(D), attn_scale(D)
    first = None
    for s, (q, k, v) in enumerate(steps):
        print(f"[gpu] mask reuse step {s} N={N} heads={cfg.heads}", flush=True)
        out, routed = reuse.layer(to_dev(q), to_dev(k), to_dev(v), grid, cfg.top_p, cfg.k_floor)
        rp, ci, nnz = reuse.mask
        torch.cuda.synchronize()
        assert routed == (s != 1)
        nz = int(nnz.item())
        rp_h = rp.cpu().numpy().astype(np.int64)
        ci_h = ci[:nz].cpu().numpy().astype(np.int64)
        qt, kt, vt = (O.reorder(x, T, H, W, cfg.tile, B) for x in (q, k, v))
        fresh = O.route(qt, kt, N, B, cfg.top_p, cfg.k_floor, scale)
        if routed:
            rep = O.check_mask(fresh, rp_h, ci_h, cfg.top_p, cfg.k_floor)
            assert rep.ok, rep.failures[:5]
        else:
            # the CSR of step 0, although this step's own routing keeps other blocks
            assert np.array_equal(rp_h, first[0]) and np.array_equal(ci_h, first[1])
            assert not (np.array_equal(fresh.row_ptr, rp_h) and
                        np.array_equal(fresh.col_idx, ci_h))
        if s == 0:
            first = (rp_h.copy(), ci_h.copy())
        Oref, _ = O.sparse_attn(qt, kt, vt, rp_h, ci_h, N, B, sc)
        got = O.reorder(to_bits(out), T, H, W, cfg.tile, B)
        d = np.abs(O.widen_bf16(got)[:, :, :N] - Oref[:, :, :N])
        print(f"[gpu]   routed={routed} nnz {nz}; out max-abs {d.max():.3e} "
              f"mean-abs {d.mean():.3e}", flush=True)
        assert d.max() <= 2e-2 and d.mean() <= 2e-3

