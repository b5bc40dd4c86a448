"""Attention recall of the routed masks under the 3D-tile and the Hilbert token orders
(the DFSAttn page, abstract, studies sparse attention through a lower bound on attention
recall and reorders tokens along a Hilbert curve), on sampled heads of the Wan-480p workload,
with the oracle router and exact attention (CPU).

recall(query) = the share of the query's exact softmax mass (over all N keys) that falls in
the key blocks its row keeps.  The Hilbert order keeps fewer blocks at the same p; the test
checks that its recall stays within 1 % of the tile order's and prints both."""
import math

import numpy as np

import oracle as O
from workloads import CONFIGS, gen_qkv


def _recall_and_sparsity(q, k, cfg, pi, qblocks):
    T, H, W, B = cfg.T, cfg.H, cfg.W, cfg.block
    qt = O.reorder(q, T, H, W, cfg.tile, B, pi=pi)
    kt = O.reorder(k, T, H, W, cfg.tile, B, pi=pi)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    rt = O.route(qt, kt, cfg.N, B, cfg.top_p, cfg.k_floor, scale)
    n = O.num_blocks(cfg.N, B)
    qf, kf = O.widen_bf16(qt), O.widen_bf16(kt)
    rec = []
    for hh in range(qt.shape[1]):
        for i in qblocks:
            lo, hi = i * B, min((i + 1) * B, cfg.N)
            lg = scale * (qf[0, hh, lo:hi] @ kf[0, hh, :cfg.N].T)
            w = np.exp(lg - lg.max(axis=1, keepdims=True))
            w /= w.sum(axis=1, keepdims=True)
            r = hh * n + i
            keep = np.zeros(cfg.N, bool)
            for j in rt.col_idx[rt.row_ptr[r]:rt.row_ptr[r + 1]]:
                keep[j * B:min((j + 1) * B, cfg.N)] = True
            rec.append(w[:, keep].sum(axis=1))
    sparsity = 1 - rt.row_ptr[-1] / (qt.shape[1] * n * n)
    return float(np.mean(np.concatenate(rec))), sparsity


def test_hilbert_order_recall_on_wan480p():
    cfg = CONFIGS["wan480p"]
    q, k, _ = gen_qkv(cfg, heads=[0, 13, 27])
    qblocks = range(0, O.num_blocks(cfg.N, cfg.block), 16)
    r_tile, s_tile = _recall_and_sparsity(q, k, cfg, None, qblocks)
    r_hil, s_hil = _recall_and_sparsity(q, k, cfg, O.hilbert_perm(cfg.T, cfg.H, cfg.W), qblocks)
    print(f"tile: sparsity {s_tile:.4f} recall {r_tile:.4f}; "
          f"hilbert: sparsity {s_hil:.4f} recall {r_hil:.4f}")
    assert s_hil > s_tile
    assert r_hil >= r_tile - 0.01
