"""Pins of the oracle's block scoring and Top-p / Top-k routing (CPU only)."""
import itertools
import math
import os

import numpy as np
from scipy.special import softmax

import oracle as O
from oracle.check import check_row


def _golden_rows(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "route_hand.txt")) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            s, p, kf, cols = [x.strip() for x in line.split("|")]
            s = [math.log(float(t[3:])) for t in s.split()]
            rows.append((np.array(s), float(p), int(kf), [int(c) for c in cols.split()]))
    return rows


def test_hand_worked_rows(golden_dir):
    rows = _golden_rows(golden_dir)
    assert len(rows) == 12
    for s, p, kf, cols in rows:
        r = O.route_row(s, p, kf)
        assert r.cols.tolist() == cols, (s, p, kf)
        assert r.count == len(cols)


def test_mass_is_library_softmax():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((4, 9)) * 5
    P = O.block_mass(s)
    assert np.allclose(P, softmax(s, axis=-1), rtol=1e-14, atol=0)
    assert np.allclose(P.sum(-1), 1.0, atol=1e-15)


def test_scores_symmetry_and_scale():
    rng = np.random.default_rng(4)
    a = rng.standard_normal((1, 2, 6, 5))
    b = rng.standard_normal((1, 2, 6, 5))
    s = O.block_scores(a, a, 0.5)
    assert np.allclose(s, np.swapaxes(s, -1, -2), rtol=0, atol=1e-15)
    assert np.allclose(O.block_scores(3 * a, b, 0.5), 3 * O.block_scores(a, b, 0.5),
                       rtol=1e-14)
    # one explicit entry
    assert math.isclose(O.block_scores(a, b, 0.5)[0, 1, 2, 4],
                        0.5 * sum(a[0, 1, 2, d] * b[0, 1, 4, d] for d in range(5)),
                        rel_tol=1e-14)


def test_p_one_dense_and_floor_ge_n_dense():
    rng = np.random.default_rng(5)
    for _ in range(20):
        s = rng.standard_normal(11) * 4
        assert O.route_row(s, 1.0, 1).cols.tolist() == list(range(11))
        assert O.route_row(s, 0.3, 11).cols.tolist() == list(range(11))
        assert O.route_row(s, 0.3, 50).cols.tolist() == list(range(11))


def test_p_zero_is_stable_argsort_topk():
    rng = np.random.default_rng(6)
    for kf in (1, 2, 5):
        for _ in range(20):
            s = np.round(rng.standard_normal(12) * 2, 1)        # plenty of exact ties
            expect = np.sort(np.argsort(-s, kind="stable")[:kf])
            assert O.route_row(s, 0.0, kf).cols.tolist() == expect.tolist()


def test_zero_queries_uniform_closed_form():
    # Q == 0 gives all-zero scores, uniform mass 1/n and index order; for p*n not an
    # integer the Top-p count is ceil(p*n): Tiny (n_blk = 8): p=0.6 -> 5, p=0.9 -> 8.
    N, B, D = 512, 64, 8
    q = np.zeros((1, 1, N, D))
    k = np.random.default_rng(7).standard_normal((1, 1, N, D))
    for p, kf, want in [(0.6, 2, 5), (0.9, 2, 8), (0.3, 1, 3), (0.3, 6, 6), (0.01, 1, 1)]:
        rt = O.route(q, k, N, B, p, kf, 0.125)
        assert rt.rows[0].cols.tolist() == list(range(want)), p


def test_bruteforce_minimal_subsets():
    # The Top-p count must be the least number of blocks whose mass can reach p (greedy by
    # mass is optimal), the kept set must carry the largest mass of any set of that size,
    # and the floor raises the count.  Enumerate every subset of small rows.
    rng = np.random.default_rng(8)
    tested = 0
    for trial in range(300):
        n = int(rng.integers(1, 8))
        s = rng.standard_normal(n) * rng.uniform(0.5, 4)
        p = float(rng.uniform(0.05, 0.99))
        kf = int(rng.integers(1, n + 1))
        P = softmax(s)
        sums = {}
        for r in range(1, n + 1):
            sums[r] = max(sum(P[list(c)]) for c in itertools.combinations(range(n), r))
        if any(abs(v - p) < 1e-9 for v in sums.values()):
            continue
        kstar = min(r for r in range(1, n + 1) if sums[r] >= p)
        rr = O.route_row(s, p, kf)
        assert rr.k_p == kstar
        c = min(n, max(kstar, kf))
        assert rr.count == c
        assert math.isclose(P[rr.cols].sum(), sums[c], rel_tol=1e-12)
        tested += 1
    assert tested > 250


def test_fp64_shortfall_keeps_all():
    # 14 equal blocks: the fp64 running sum of the mass stops at 1 - 3 ulp, so a p between
    # that sum and 1 is never reached and every block is kept
    s = np.zeros(14)
    rr = O.route_row(s, 0.9999999999999998, 1)
    assert rr.cum[-1] < 0.9999999999999998
    assert rr.count == 14 and rr.k_p == 14


def test_route_csr_layout():
    rng = np.random.default_rng(9)
    N, B, D = 200, 16, 4                                      # 13 blocks, last one short
    q = rng.standard_normal((2, 3, 208, D))
    k = rng.standard_normal((2, 3, 208, D))
    rt = O.route(q, k, N, B, 0.7, 2, 0.5)
    assert rt.row_ptr.shape == (2 * 3 * 13 + 1,)
    assert rt.row_ptr[0] == 0 and np.all(np.diff(rt.row_ptr) >= 2)
    for r in range(78):
        cols = rt.col_idx[rt.row_ptr[r]:rt.row_ptr[r + 1]]
        assert np.all(np.diff(cols) > 0)
    # padding rows of the input do not matter
    q2, k2 = q.copy(), k.copy()
    q2[:, :, N:] = 99.0
    k2[:, :, N:] = -99.0
    rt2 = O.route(q2, k2, N, B, 0.7, 2, 0.5)
    assert np.array_equal(rt.col_idx, rt2.col_idx)


# --- the acceptance checker must catch planted mistakes and accept legal alternatives ----
def _row(s, p, kf):
    return s, O.route_row(s, p, kf)


def test_checker_exact_and_planted_errors():
    s, rr = _row(np.array([3.0, 1.0, 2.0, 0.5, -1.0, 2.5]), 0.8, 1)
    assert check_row(s, rr, 0.8, 1, rr.cols) == "exact"
    wrong = sorted(set(rr.cols.tolist()) - {int(rr.order[0])} | {int(rr.order[-1])})
    assert check_row(s, rr, 0.8, 1, wrong).startswith("fail")
    assert check_row(s, rr, 0.8, 1, rr.cols[:-1]).startswith("fail")       # count, no slack
    assert check_row(s, rr, 0.8, 1, rr.cols[::-1]).startswith("fail")      # not ascending


def test_checker_accepts_tie_swaps_only():
    s = np.array([2.0, 1.0, 1.0 + 1e-9, 0.0])       # blocks 1 and 2 tie within 1e-6
    rr = O.route_row(s, 0.0, 2)                     # top-2 = {0, 2}
    assert rr.cols.tolist() == [0, 2]
    assert check_row(s, rr, 0.0, 2, [0, 1]) == "tie"
    assert check_row(s, rr, 0.0, 2, [0, 3]).startswith("fail")
    assert check_row(s, rr, 0.0, 2, [1, 2]).startswith("fail")


def test_checker_count_slack_near_threshold():
    s = np.array([math.log(4), math.log(2), 0.0, 0.0])    # cum 0.5 0.75 0.875 1
    rr = O.route_row(s, 0.75 + 5e-7, 1)                   # oracle needs 3 blocks
    assert rr.count == 3
    assert check_row(s, rr, 0.75 + 5e-7, 1, [0, 1]) == "count"    # within 1e-6 of p
    rr = O.route_row(s, 0.75 + 5e-6, 1)
    assert check_row(s, rr, 0.75 + 5e-6, 1, [0, 1]).startswith("fail")
    rr = O.route_row(s, 0.75 - 5e-7, 1)                   # oracle keeps 2
    assert rr.count == 2
    assert check_row(s, rr, 0.75 - 5e-7, 1, [0, 1, 2]) == "count"
    rr = O.route_row(s, 0.5, 3)                           # floor sets the count: no slack
    assert check_row(s, rr, 0.5, 3, [0, 1]).startswith("fail")
