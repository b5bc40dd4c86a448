"""Pins of the oracle's periodic-stripe masks (reading of the PSA page's six-parameter mask,
"Approach"): hand-worked cases, closed forms, and the binding's host-side checks."""
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stripe_hand.txt")


def _cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        head, *rest = line.split(None, 1)
        if head == "case":
            g, t, b, p = rest[0].split("|")
            cur = dict(grid=tuple(map(int, g.split())), tile=tuple(map(int, t.split())),
                       B=int(b), params=tuple(map(int, p.split())), coords=None, rows=[])
            cases.append(cur)
        elif head == "coords":
            cur["coords"] = [tuple(map(int, c.split(":"))) for c in rest[0].split()]
        elif head == "row":
            cur["rows"].append([int(x) for x in rest[0].split()] if rest else [])
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "x".join(map(str, c["grid"])))
def test_hand_worked_masks(case):
    T, H, W = case["grid"]
    bt, bs = O.block_coords(T, H, W, case["tile"], case["B"])
    assert list(zip(bt.tolist(), bs.tolist())) == case["coords"]
    rp, ci = O.stripe_mask(T, H, W, case["tile"], case["B"], [case["params"]])
    got = [ci[rp[i]:rp[i + 1]].tolist() for i in range(len(rp) - 1)]
    assert got == case["rows"]


def test_full_width_is_dense():
    """Tw = Ts and Sw = Ss keep every block, whatever the offsets."""
    T, H, W, tile, B = 21, 30, 52, (4, 4, 8), 128
    n = O.num_blocks(T * H * W, B)
    rp, ci = O.stripe_mask(T, H, W, tile, B, [(3, 5, 3, 7, -2, 7), (1, 0, 1, 1, 0, 1)])
    assert rp[-1] == 2 * n * n
    assert np.array_equal(ci[:n], np.arange(n))


def test_same_spatial_tile_closed_form():
    """Aligned grid (every block one full tile): Ts = Tw = 1, Sw = 1, So = 0 and a period
    larger than any spatial index keep exactly the blocks of the same spatial tile, one per
    temporal slab: nT per row, at stride nS."""
    T, H, W, tile, B = 8, 16, 32, (2, 4, 8), 64
    nT, nS = 4, 4 * 4
    rp, ci = O.stripe_mask(T, H, W, tile, B, [(1, 0, 1, 1, 0, 1000)])
    counts = np.diff(rp)
    assert np.all(counts == nT)
    for i in (0, 5, nS + 3, 3 * nS + 15):
        assert ci[rp[i]:rp[i + 1]].tolist() == [i % nS + k * nS for k in range(nT)]


def test_diagonal_kept_with_zero_offsets_and_periodicity():
    T, H, W, tile, B = 9, 20, 24, (2, 4, 4), 64
    bt, bs = O.block_coords(T, H, W, tile, B)
    keep = O.stripe_keep(bt, bs, (2, 0, 5, 3, 0, 6))
    assert np.all(np.diag(keep))
    # shifting the offset by a whole period changes nothing
    assert np.array_equal(keep, O.stripe_keep(bt, bs, (2, 5, 5, 3, -6, 6)))


@pytest.mark.parametrize("p", [(0, 0, 1, 1, 0, 1), (2, 0, 1, 1, 0, 1), (1, 0, 1, 3, 0, 2),
                               (1, 0, 0, 1, 0, 1)])
def test_invalid_parameters_rejected(p):
    with pytest.raises(ValueError):
        O.stripe_mask(2, 4, 4, (1, 2, 2), 4, [p])
