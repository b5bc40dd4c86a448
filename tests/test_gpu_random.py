"""GPU parity on a seeded sweep of small configurations: grid, tile, head_dim, block, heads,
batch, Top-p, Top-k floor and token order drawn from a fixed seed, each run through the
whole path (reorder, routing, attention, inverse) and checked against the oracle with the
bars of the other parity tests (reorder and inverse bit-exact, every mask row accepted, fp64
scores within 1e-12 of the row's largest, output max-abs 2e-2 / mean-abs 2e-3, LSE 1e-3)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import Config, gen_qkv

from gpu_common import attn_scale, bf16_f64, to_bits, to_dev

pytestmark = pytest.mark.gpu


def _draw(n_cases=12, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        D = int(rng.choice([64, 128]))
        B = int(rng.choice([64, 128]))
        tile = tuple(int(x) for x in rng.choice([1, 2, 4, 8], size=3))
        cases.append(dict(
            T=int(rng.integers(1, 9)), H=int(rng.integers(3, 33)), W=int(rng.integers(3, 33)),
            D=D, B=B, tile=tile, heads=int(rng.integers(1, 4)), batch=int(rng.integers(1, 3)),
            top_p=float(rng.choice([0.5, 0.8, 0.9, 0.95, 1.0])),
            k_floor=int(rng.choice([1, 2, 4])), order=str(rng.choice(["tile", "hilbert"])),
            seed=1000 + i))
    return cases


CASES = _draw()


@pytest.mark.parametrize("c", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_random_config(c):
    T, H, W, D, B = c["T"], c["H"], c["W"], c["D"], c["B"]
    print(f"[gpu] random {c}", flush=True)
    parts = [gen_qkv(Config("rnd", T, H, W, c["heads"], D, B, c["tile"], c["top_p"],
                            c["k_floor"], c["seed"] + 17 * bi),
                     gains=np.full(c["heads"], 1.5)) for bi in range(c["batch"])]
    q, k, v = (np.concatenate([p[t] for p in parts], axis=0) for t in range(3))
    grid = bsa.Grid(T, H, W, c["tile"], B)
    pi = None
    if c["order"] == "hilbert":
        grid = grid.with_order(bsa.hilbert_order(grid))
        pi = O.hilbert_perm(T, H, W)
    N, n = T * H * W, grid.n_blk
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    q_t, k_t, v_t = bsa.reorder(tq, grid), bsa.reorder(tk, grid), bsa.reorder(tv, grid)
    scale = 1.0 / math.sqrt(D)
    rp, ci, nnz, S = bsa.score_and_route(q_t, k_t, grid, c["top_p"], c["k_floor"], scale,
                                         return_scores=True)
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, sc)
    out = bsa.reorder(out_t, grid, inverse=True)
    torch.cuda.synchronize()
    refs = [O.reorder(x, T, H, W, c["tile"], B, pi=pi) for x in (q, k, v)]
    for t, ref in zip((q_t, k_t, v_t), refs):
        assert np.array_equal(to_bits(t), ref)
    ref = O.route(refs[0], refs[1], N, B, c["top_p"], c["k_floor"], scale)
    s_err = np.abs(S.cpu().numpy() - ref.scores).max(axis=-1) / np.maximum(
        np.abs(ref.scores).max(axis=-1), 1e-300)
    assert s_err.max() <= 1e-12
    nz = int(nnz.item())
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:nz].cpu().numpy().astype(np.int64)
    rep = O.check_mask(ref, rp_h, ci_h, c["top_p"], c["k_floor"])
    assert rep.rows == c["batch"] * c["heads"] * n and rep.ok, rep.failures[:5]
    Oref, Lref = O.sparse_attn(refs[0], refs[1], refs[2], rp_h, ci_h, N, B, sc)
    d = np.abs(bf16_f64(out_t)[:, :, :N] - Oref[:, :, :N])
    print(f"[gpu]   n_blk {n} nnz {nz}; out max-abs {d.max():.3e} mean-abs {d.mean():.3e}",
          flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert np.abs(lse.cpu().numpy()[:, :, :N] - Lref[:, :, :N]).max() <= 1e-3
    assert np.all(to_bits(out_t)[:, :, N:] == 0)
    assert np.array_equal(to_bits(out), O.inverse_reorder(to_bits(out_t), T, H, W, c["tile"],
                                                          pi=pi))
