"""Pins of the oracle's 3D-tile token order and block pooling (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import CONFIGS, bf16_bits_from_f64

GRIDS = [(c.T, c.H, c.W, c.tile) for c in CONFIGS.values()] + [(3, 5, 7, (2, 2, 3)),
                                                                 (1, 1, 1, (4, 4, 8))]


@pytest.mark.parametrize("T,H,W,tile", GRIDS)
def test_closed_form_equals_sort_and_is_bijection(T, H, W, tile):
    pi = O.tile_perm(T, H, W, tile)
    assert np.array_equal(pi, O.tile_perm_by_sort(T, H, W, tile))
    assert np.array_equal(np.sort(pi), np.arange(T * H * W))


def _golden_orders(golden_dir):
    out = []
    with open(os.path.join(golden_dir, "tile_order_hand.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, tail = line.split(":")
            T, H, W, a, b, c = map(int, head.split())
            out.append(((T, H, W, (a, b, c)), list(map(int, tail.split()))))
    return out


def test_hand_enumerated_orders(golden_dir):
    cases = _golden_orders(golden_dir)
    assert len(cases) == 3
    for (T, H, W, tile), order in cases:
        pi = O.tile_perm(T, H, W, tile)
        got = np.empty_like(pi)
        got[pi] = np.arange(pi.size)            # position -> raster index
        assert got.tolist() == order, (T, H, W, tile)


def test_tiny_block_map():
    # Tiny (2x16x16, tile 4x4x4, B=64): frames 0-1 form one truncated slab of 2x4x4 = 32-token
    # tiles, so each block is two tiles adjacent along w: block(t,h,w) = 2*(h//4) + (w//4)//2.
    c = CONFIGS["tiny"]
    pi = O.tile_perm(c.T, c.H, c.W, c.tile)
    t, h, w = np.meshgrid(np.arange(c.T), np.arange(c.H), np.arange(c.W), indexing="ij")
    expect = (2 * (h // 4) + (w // 4) // 2).ravel()
    assert np.array_equal(pi // c.block, expect)


def test_small_block_map():
    # Small (5x16x24, tile 4x4x4, B=64): blocks 0..23 are the 24 full tiles of frames 0-3 in
    # (ih, iw) order; blocks 24..29 hold frame 4 (a truncated slab of 1x4x4 tiles).
    c = CONFIGS["small"]
    pi = O.tile_perm(c.T, c.H, c.W, c.tile)
    t, h, w = np.meshgrid(np.arange(c.T), np.arange(c.H), np.arange(c.W), indexing="ij")
    t, h, w = t.ravel(), h.ravel(), w.ravel()
    blk = pi // c.block
    full = t < 4
    assert np.array_equal(blk[full], (h // 4 * 6 + w // 4)[full])
    assert set(blk[~full].tolist()) == set(range(24, 30))
    assert np.all(np.bincount(blk) == 64)


def test_reorder_inverse_roundtrip_and_padding():
    rng = np.random.default_rng(0)
    T, H, W, tile, B = 3, 5, 7, (2, 2, 3), 8              # N = 105, Npad = 112
    x = rng.standard_normal((2, T * H * W, 3, 4))
    xt = O.reorder(x, T, H, W, tile, B)
    assert xt.shape == (2, 3, 112, 4)
    assert np.all(xt[:, :, 105:] == 0)
    assert np.array_equal(O.inverse_reorder(xt, T, H, W, tile), x)
    # each token lands at pi(n) for every batch and head
    pi = O.tile_perm(T, H, W, tile)
    assert np.array_equal(xt[1, 2, pi[17]], x[1, 17, 2])


def test_pool_exact_and_short_last_block():
    rng = np.random.default_rng(1)
    N, B, D = 37, 8, 3                                     # last block holds 5 real tokens
    bits = bf16_bits_from_f64(rng.standard_normal((1, 1, 40, D)) * 3)
    bits[:, :, N:] = 0
    x = O.widen_bf16(bits)
    got = O.pool(x, N, B)
    assert got.shape == (1, 1, 5, D)
    for j in range(5):
        lo, hi = j * B, min((j + 1) * B, N)
        for d in range(D):
            exact = sum(Fraction(float(v)) for v in x[0, 0, lo:hi, d]) / (hi - lo)
            # fp64 sum of <= 128 bf16 values of moderate range is exact; one division rounding
            assert got[0, 0, j, d] == float(exact)


def test_pool_constant_blocks():
    N, B, D = 20, 8, 2
    x = np.zeros((1, 2, 24, D))
    for j in range(3):
        x[:, :, j * B:min((j + 1) * B, N)] = j + 0.25
    got = O.pool(x, N, B)
    assert np.array_equal(got[0, 0, :, 0], [0.25, 1.25, 2.25])
