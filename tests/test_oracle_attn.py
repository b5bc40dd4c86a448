"""Pins of the oracle's exact block-sparse attention (CPU only).

Independent anchors: PyTorch's own scaled_dot_product_attention on the CPU in float64 (a
library routine, with and without a boolean mask), closed forms (V = 1, K = 0, a two-key
hand example), SciPy's logsumexp, and invariances of the method (token permutation at
p = 1, shuffles inside blocks)."""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as O
from workloads import get_config, gen_qkv


def _sdpa(q, k, v, scale, mask=None):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m,
                                                            scale=scale).numpy()


def _cfg_inputs(name):
    cfg = get_config(name)
    q, k, v = gen_qkv(cfg)
    B = cfg.block
    qt, kt, vt = (O.reorder(O.widen_bf16(x), cfg.T, cfg.H, cfg.W, cfg.tile, B)
                  for x in (q, k, v))
    return cfg, (q, k, v), (qt, kt, vt)


def test_hand_two_keys():
    # one query, two keys with logits ln 3 and 0: weights 3/4 and 1/4
    q = np.array([[math.log(3.0), 0.0]])
    k = np.array([[1.0, 0.0], [0.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    qt, kt, vt = (x.reshape(1, 1, *x.shape) for x in (np.vstack([q, q]), k, v))
    row_ptr = np.array([0, 2, 4])
    col_idx = np.array([0, 1, 0, 1])
    Ot, LSE = O.sparse_attn(qt, kt, vt, row_ptr, col_idx, N=2, B=1, scale=1.0)
    assert np.allclose(Ot[0, 0, 0], [0.75, 0.25], atol=1e-15)
    assert math.isclose(LSE[0, 0, 0], math.log(4.0), rel_tol=1e-15)


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_block_gather_equals_masked_dense_and_library(name):
    cfg, _, (qt, kt, vt) = _cfg_inputs(name)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    rt = O.route(qt, kt, cfg.N, cfg.block, cfg.top_p, cfg.k_floor, scale)
    Og, Lg = O.sparse_attn(qt, kt, vt, rt.row_ptr, rt.col_idx, cfg.N, cfg.block, scale)
    Od, Ld = O.masked_dense_attn(qt, kt, vt, rt.row_ptr, rt.col_idx, cfg.N, cfg.block, scale)
    N = cfg.N
    assert np.max(np.abs(Og[:, :, :N] - Od[:, :, :N])) < 1e-12
    assert np.max(np.abs(Lg[:, :, :N] - Ld[:, :, :N])) < 1e-12
    # library: torch SDPA with the block mask expanded to tokens
    n = O.num_blocks(N, cfg.block)
    Mb = O.block_mask_dense(rt.row_ptr, rt.col_idx, 1, cfg.heads, n)
    blk = np.arange(N) // cfg.block
    mask = Mb[:, :, blk[:, None], blk[None, :]]
    ref = _sdpa(qt[:, :, :N], kt[:, :, :N], vt[:, :, :N], scale, mask)
    assert np.max(np.abs(Og[:, :, :N] - ref)) < 1e-12
    # LSE is the log-sum-exp of the allowed logits
    logits = scale * np.einsum("bhqd,bhkd->bhqk", qt[:, :, :N], kt[:, :, :N])
    lse = logsumexp(np.where(mask, logits, -np.inf), axis=-1)
    assert np.max(np.abs(Lg[:, :, :N] - lse)) < 1e-12


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_p_one_is_dense_and_permutation_invariant(name):
    cfg, (q, k, v), (qt, kt, vt) = _cfg_inputs(name)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    out, rt, Ot, _ = O.layer(q, k, v, cfg.T, cfg.H, cfg.W, cfg.tile, cfg.block, 1.0,
                             cfg.k_floor, scale)
    n = O.num_blocks(cfg.N, cfg.block)
    assert rt.nnz == cfg.heads * n * n
    dense = O.dense_attn_raster(q, k, v, scale)
    assert np.max(np.abs(out - dense)) < 1e-12
    ref = _sdpa(*(np.transpose(O.widen_bf16(x), (0, 2, 1, 3)) for x in (q, k, v)), scale)
    assert np.max(np.abs(np.transpose(out, (0, 2, 1, 3)) - ref)) < 1e-12


def test_v_one_and_k_zero_closed_forms():
    rng = np.random.default_rng(11)
    N, B, D = 50, 8, 6                                            # 7 blocks, last one short
    Npad = 56
    qt = rng.standard_normal((1, 2, Npad, D))
    kt = rng.standard_normal((1, 2, Npad, D))
    vt = rng.standard_normal((1, 2, Npad, D))
    rt = O.route(qt, kt, N, B, 0.5, 2, 0.4)
    Ot, _ = O.sparse_attn(qt, kt, np.ones_like(vt), rt.row_ptr, rt.col_idx, N, B, 0.4)
    assert np.allclose(Ot[:, :, :N], 1.0, rtol=0, atol=1e-14)
    # K == 0: uniform weights over the real keys of the selected blocks
    Ot, LSE = O.sparse_attn(qt, np.zeros_like(kt), vt, rt.row_ptr, rt.col_idx, N, B, 0.4)
    n = O.num_blocks(N, B)
    for h in range(2):
        for i in range(n):
            r = h * n + i
            keys = [u for j in rt.col_idx[rt.row_ptr[r]:rt.row_ptr[r + 1]]
                    for u in range(j * B, min((j + 1) * B, N))]
            lo, hi = i * B, min((i + 1) * B, N)
            assert np.allclose(Ot[0, h, lo:hi], vt[0, h, keys].mean(axis=0), atol=1e-14)
            assert np.allclose(LSE[0, h, lo:hi], math.log(len(keys)), atol=1e-14)


def test_shuffle_inside_blocks():
    # Permuting tokens inside each block leaves pooled means, hence the mask, unchanged,
    # and permutes the output rows the same way.
    cfg, _, (qt, kt, vt) = _cfg_inputs("tiny")
    scale = 0.125
    rng = np.random.default_rng(12)
    perm = np.concatenate([j * 64 + rng.permutation(64) for j in range(8)])
    rt = O.route(qt, kt, cfg.N, 64, cfg.top_p, cfg.k_floor, scale)
    rs = O.route(qt[:, :, perm], kt[:, :, perm], cfg.N, 64, cfg.top_p, cfg.k_floor, scale)
    assert np.array_equal(rt.row_ptr, rs.row_ptr) and np.array_equal(rt.col_idx, rs.col_idx)
    O1, _ = O.sparse_attn(qt, kt, vt, rt.row_ptr, rt.col_idx, cfg.N, 64, scale)
    O2, _ = O.sparse_attn(qt[:, :, perm], kt[:, :, perm], vt[:, :, perm], rs.row_ptr,
                          rs.col_idx, cfg.N, 64, scale)
    assert np.max(np.abs(O1[:, :, perm] - O2)) < 1e-12


def test_attention_rows_sum_to_one():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((5, 4)) * 3
    k = rng.standard_normal((9, 4)) * 3
    logits = 0.7 * q @ k.T
    _, lse = O.bsa_oracle._attend(q, k, np.eye(9), 0.7)
    w = np.exp(logits - lse[:, None])
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)


def test_subset_heads_and_rows():
    cfg, _, (qt, kt, vt) = _cfg_inputs("small")
    scale = 0.125
    rt = O.route(qt, kt, cfg.N, cfg.block, cfg.top_p, cfg.k_floor, scale)
    full, _ = O.sparse_attn(qt, kt, vt, rt.row_ptr, rt.col_idx, cfg.N, cfg.block, scale)
    part, _ = O.sparse_attn(qt, kt, vt, rt.row_ptr, rt.col_idx, cfg.N, cfg.block, scale,
                            heads=[3], qblocks=[0, 29])
    m = ~np.isnan(part)
    assert m.sum() == 2 * 64 * cfg.head_dim
    assert np.array_equal(part[m], full[m])
