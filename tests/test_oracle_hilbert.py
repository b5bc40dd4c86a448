"""Pins of the oracle's Hilbert-curve token order (reading of the DFSAttn page's Hilbert
reordering): the defining properties of a 3D Hilbert curve on full cubes, and the order of a
grid embedded in its cube."""
import numpy as np
import pytest

import oracle as O


def _cube(b):
    s = 1 << b
    t, h, w = np.meshgrid(np.arange(s), np.arange(s), np.arange(s), indexing="ij")
    return t.ravel(), h.ravel(), w.ravel()


@pytest.mark.parametrize("b", [1, 2, 3, 4, 5])
def test_curve_is_a_bijection_with_unit_steps(b):
    t, h, w = _cube(b)
    idx = O.hilbert_index(t, h, w, b)
    assert np.array_equal(np.sort(idx), np.arange(8 ** b))
    o = np.argsort(idx)
    c = np.stack([t[o], h[o], w[o]], 1)
    assert np.all(np.abs(np.diff(c, axis=0)).sum(axis=1) == 1)    # face neighbours
    assert idx[0] == 0                                             # starts at the origin


@pytest.mark.parametrize("b,j", [(3, 1), (4, 1), (4, 2), (4, 3), (5, 2)])
def test_aligned_subcubes_are_contiguous(b, j):
    """The recursive property: every aligned sub-cube of side 2^j is one run of 8^j indices."""
    t, h, w = _cube(b)
    idx = O.hilbert_index(t, h, w, b)
    key = ((t >> j) << (2 * (b - j))) | ((h >> j) << (b - j)) | (w >> j)
    for k in np.unique(key):
        v = np.sort(idx[key == k])
        assert v[-1] - v[0] == 8 ** j - 1 and v[0] % (8 ** j) == 0


def test_embedded_grid_order():
    T, H, W = 5, 6, 11                                  # cube side 16
    assert O.cube_bits(T, H, W) == 4
    pi = O.hilbert_perm(T, H, W)
    assert np.array_equal(np.sort(pi), np.arange(T * H * W))
    order = O.hilbert_order(T, H, W)
    assert np.array_equal(pi[order], np.arange(T * H * W))
    t, h, w = order // (H * W), (order // W) % H, order % W
    idx = O.hilbert_index(t, h, w, 4)
    assert np.all(np.diff(idx) > 0)                     # positions follow the curve


def test_blocks_are_compact_on_video_grids():
    """Blocks of 128 consecutive tokens: mean bounding-box volume no larger than about twice
    the block (a 3D-tile block of 4 x 4 x 8 has volume exactly 128)."""
    T, H, W = 21, 30, 52
    order = O.hilbert_order(T, H, W)
    vols = []
    for j in range(len(order) // 128):
        n = order[j * 128:(j + 1) * 128]
        t, h, w = n // (H * W), (n // W) % H, n % W
        vols.append((np.ptp(t) + 1) * (np.ptp(h) + 1) * (np.ptp(w) + 1))
    assert np.median(vols) <= 256
