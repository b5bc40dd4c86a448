"""GPU test of the attention's online softmax at extreme logit ranges, through the C ABI.

The kernel keeps a per-row reference m (log2 units) and takes 2^(logit - m) for every key; m
is the first key block's row maximum and moves up only when a later block would overflow the
block sum (the exponential overflows fp32 at 128 and underflows below -126).  Rows here are
built so that every branch of that logic runs: logits that jump by hundreds from one key block
to the next (2^x overflows to inf against the old reference), that climb past the reference at
every block, that sit hundreds below zero, and the mirror images (first block the largest).
Q, K, V are written straight into the tiled layout (block b = rows b*B .. b*B + B - 1, pad rows
zero) and run over a dense CSR and over one with every row's columns in a rotated order.
Checked against the oracle's fp64 attention with the usual bars (output max-abs 2e-2,
mean-abs 2e-3, LSE 1e-3).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
import oracle as O
from workloads import bf16_bits_from_f64, f64_from_bf16_bits

from gpu_common import attn_scale, bf16_f64

pytestmark = pytest.mark.gpu

# per-block logit targets (log2 units) for queries of sign +1; queries of sign -1 see -T
PATTERNS = {
    "jump": [-300.0, 0.0, 250.0, -80.0, 120.0],
    "ramp": [-24.0, -12.0, 0.0, 12.0, 24.0],
    "low": [-400.0, -390.0, -410.0, -395.0, -405.0],
}


def _inputs(D, B, N, targets, seed):
    """Tiled bf16 bit patterns [1, 1, Npad, D] of Q, K, V whose logits c*q.k (c = log2(e) *
    scale) are about sign_i * targets[block of the key] plus a few log2 units of noise."""
    rng = np.random.default_rng(seed)
    nb = -(-N // B)
    Npad = nb * B
    c = np.log2(np.e) * attn_scale(D)
    u = rng.choice([-1.0, 1.0], size=D)
    sign = np.where(np.arange(N) % 2 == 0, 1.0, -1.0)
    q = sign[:, None] * u[None, :] + 0.05 * rng.standard_normal((N, D))
    gam = np.repeat(np.asarray(targets[:nb]) / (c * D), B)[:N]
    k = gam[:, None] * u[None, :] + 1.5 * rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    out = []
    for x in (q, k, v):
        t = np.zeros((1, 1, Npad, D))
        t[0, 0, :N] = x
        out.append(bf16_bits_from_f64(t))
    return out


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.bfloat16).to("cuda:0")


@pytest.mark.parametrize("pattern", sorted(PATTERNS))
@pytest.mark.parametrize("D,B,rotate", [(128, 128, False), (128, 128, True), (64, 64, False)],
                         ids=["d128", "d128_rotated", "d64"])
def test_extreme_logits(pattern, D, B, rotate):
    N = 5 * B - 37                                    # five key blocks, the last one short
    grid = bsa.Grid(1, 1, N, (1, 1, B), B)
    assert grid.n_blk == 5 and grid.Npad == 5 * B
    qb, kb, vb = _inputs(D, B, N, PATTERNS[pattern], 7 + D)
    n = grid.n_blk
    rows = []
    for i in range(n):
        cols = list(range(n))
        if rotate:
            cols = cols[i:] + cols[:i]
        rows.append(cols)
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    ci = np.concatenate(rows).astype(np.int64)
    print(f"[gpu] logit range {pattern} D={D} B={B} N={N} rotate={rotate}", flush=True)
    q_t, k_t, v_t = _dev(qb), _dev(kb), _dev(vb)
    sc = attn_scale(D)
    out_t, lse = bsa.sparse_attn_fwd(q_t, k_t, v_t,
                                     torch.from_numpy(rp.astype(np.int32)).to("cuda:0"),
                                     torch.from_numpy(ci.astype(np.int32)).to("cuda:0"),
                                     grid, sc)
    torch.cuda.synchronize()
    Oref, Lref = O.sparse_attn(qb, kb, vb, rp, ci, N, B, sc)
    got = bf16_f64(out_t)
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(lse.cpu().numpy()))
    d = np.abs(got[:, :, :N] - Oref[:, :, :N])
    dl = np.abs(lse.cpu().numpy().astype(np.float64)[:, :, :N] - Lref[:, :, :N])
    print(f"[gpu]   out max-abs {d.max():.3e} mean-abs {d.mean():.3e}; lse max-abs "
          f"{dl.max():.3e}; |lse| up to {np.abs(Lref).max():.1f}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    assert dl.max() <= 1e-3
    assert np.all(got[:, :, N:] == 0)
    # the rows really span the range the test is about
    logit = (f64_from_bf16_bits(qb)[0, 0, :N] @ f64_from_bf16_bits(kb)[0, 0, :N].T) * sc \
        * np.log2(np.e)
    if pattern == "low":
        assert np.abs(logit).min() > 300
    else:
        span = logit.max(axis=1) - logit.min(axis=1)
        assert span.min() > (40 if pattern == "ramp" else 300)
