"""Denoising-step drift of the inputs and mask reuse across steps (CPU).

* gen_qkv_steps: step 0 is the base workload byte for byte, zero drift repeats it, every step
  keeps the base distribution and two steps d apart are correlated by cos(d * drift).
* Mask reuse (the DFSAttn page, abstract, caches sparse masks; read here as reuse across
  denoising steps): with the oracle router and exact softmax on sampled Wan-480p heads, the
  recall of a mask kept from step 0 falls as the inputs drift away, while a freshly routed
  mask keeps its recall.
* The binding's MaskReuse / layer(mask=...) argument checks (host side, no GPU)."""
import math

import numpy as np
import pytest

import oracle as O
from workloads import CONFIGS, gen_qkv, gen_qkv_steps, f64_from_bf16_bits


def test_step_zero_is_the_base_workload():
    cfg = CONFIGS["small"]
    base = gen_qkv(cfg)
    (s0, s2) = gen_qkv_steps(cfg, [0, 2], drift=0.1)
    for a, b in zip(base, s0):
        assert np.array_equal(a, b)
    assert not np.array_equal(base[0], s2[0])
    for a, b in zip(gen_qkv_steps(cfg, [3], drift=0.0)[0], base):
        assert np.array_equal(a, b)


def test_step_correlation_and_stationarity():
    cfg = CONFIGS["small"]
    drift = 0.3
    S = [0, 1, 3, 5]
    steps = gen_qkv_steps(cfg, S, drift=drift)
    v0 = f64_from_bf16_bits(steps[0][2]).ravel()
    for s, (_, _, v) in zip(S, steps):
        vs = f64_from_bf16_bits(v).ravel()
        rho = float(np.dot(v0, vs) / math.sqrt(np.dot(v0, v0) * np.dot(vs, vs)))
        assert abs(rho - math.cos(s * drift)) < 0.03, (s, rho)
        assert abs(vs.var() / v0.var() - 1.0) < 0.05, s


def test_drift_angle_limit():
    with pytest.raises(ValueError):
        gen_qkv_steps(CONFIGS["tiny"], [0, 8], drift=0.4)


def _recall(qf, kf, rp, ci, N, B, n, scale, qblocks):
    rec = []
    for hh in range(qf.shape[1]):
        for i in qblocks:
            lo, hi = i * B, min((i + 1) * B, N)
            lg = scale * (qf[0, hh, lo:hi] @ kf[0, hh, :N].T)
            w = np.exp(lg - lg.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            r = hh * n + i
            keep = np.zeros(N, bool)
            for j in ci[rp[r]:rp[r + 1]]:
                keep[j * B:min((j + 1) * B, N)] = True
            rec.append(w[:, keep].sum(axis=1))
    return float(np.mean(np.concatenate(rec)))


def test_stale_mask_recall_falls_with_drift():
    cfg = CONFIGS["wan480p"]
    B, N = cfg.block, cfg.N
    n = O.num_blocks(N, B)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    S = [0, 2, 4, 8]                                   # angles 0, 0.2, 0.4, 0.8 rad
    steps = gen_qkv_steps(cfg, S, drift=0.1, heads=[0, 13])
    qblocks = range(0, n, 16)
    first, fresh, stale = None, [], []
    for q, k, _ in steps:
        qt, kt = (O.reorder(x, cfg.T, cfg.H, cfg.W, cfg.tile, B) for x in (q, k))
        rt = O.route(qt, kt, N, B, cfg.top_p, cfg.k_floor, scale)
        if first is None:
            first = rt
        qf, kf = O.widen_bf16(qt), O.widen_bf16(kt)
        fresh.append(_recall(qf, kf, rt.row_ptr, rt.col_idx, N, B, n, scale, qblocks))
        stale.append(_recall(qf, kf, first.row_ptr, first.col_idx, N, B, n, scale, qblocks))
    print("recall fresh", np.round(fresh, 4), "stale", np.round(stale, 4))
    assert all(a > b for a, b in zip(stale, stale[1:]))         # falls with every step
    assert all(s <= f + 2e-3 for s, f in zip(stale, fresh))
    assert stale[-1] < fresh[-1] - 0.02
    assert min(fresh) > 0.88


def test_mask_reuse_host_checks():
    bsa = pytest.importorskip("block_sparse_attention_gather_amd")
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        bsa.MaskReuse(0)
    grid = bsa.Grid(2, 8, 16, (2, 4, 8), 64)
    x = torch.zeros((1, grid.N, 1, 64), dtype=torch.bfloat16)
    rp = torch.zeros(2 * grid.n_blk + 1, dtype=torch.int32)     # a mask of a 2-head call
    with pytest.raises(ValueError):
        bsa.layer(x, x, x, grid, 0.9, 2, mask=(rp, rp, rp[:1]))
