"""Acceptance checks that compare a routed mask and an attention output with the oracle.

TEST INFRASTRUCTURE ONLY (see bsa_oracle.py).

Mask rule.  Several masks can be correct when scores tie or when the block-mass prefix sits
on the Top-p threshold to within rounding, so a candidate row set S' of size c' is accepted
iff (a) c' equals the oracle count c, or differs by one where rounding of the cumulative mass
near p (within 1e-6) could explain it and the floor is not what set the count, and (b) S'
is a top-c' set of the oracle's fp64 scores once entries whose scores tie with the c'-th
score (relative gap <= 1e-6) may be exchanged.  Everything else is a failure.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

from .bsa_oracle import RowRoute, Routing

TIE_REL = 1e-6
MASS_TOL = 1e-6


def _tie(a, b):
    return np.abs(a - b) <= TIE_REL * np.maximum(np.abs(a), np.abs(b))


def check_row(s_row, rr: RowRoute, top_p: float, k_floor: int, cand) -> str:
    """Classify one candidate row: 'exact', 'tie', 'count', or 'fail:<reason>'."""
    cand = np.asarray(cand, dtype=np.int64)
    n = s_row.size
    c, cp = rr.count, cand.size
    if cp and (np.any(np.diff(cand) <= 0) or cand[0] < 0 or cand[-1] >= n):
        return "fail:columns not strictly ascending / out of range"
    relaxed_count = False
    if cp != c:
        ok = False
        if cp == c - 1 and c == rr.k_p and c > k_floor and 0 < top_p < 1:
            ok = rr.cum[c - 2] >= top_p - MASS_TOL if c >= 2 else False
        elif cp == c + 1 and c == rr.k_p and c >= k_floor and c < n and 0 < top_p < 1:
            ok = rr.cum[c - 1] < top_p + MASS_TOL
        if not ok:
            return f"fail:count {cp} vs oracle {c}"
        relaxed_count = True
    if np.array_equal(cand, np.sort(rr.order[:cp])):
        return "count" if relaxed_count else "exact"
    if cp == 0:
        return "fail:empty"
    v = s_row[rr.order[cp - 1]]                  # c'-th largest score
    tied = _tie(s_row, v)
    must_in = (s_row > v) & ~tied
    must_out = (s_row < v) & ~tied
    inset = np.zeros(n, dtype=bool)
    inset[cand] = True
    if np.any(must_in & ~inset):
        return "fail:missing a block whose score beats the cut"
    if np.any(must_out & inset):
        return "fail:holds a block whose score is below the cut"
    return "count" if relaxed_count else "tie"


@dataclass
class MaskReport:
    rows: int = 0
    exact: int = 0
    tie: int = 0
    count: int = 0
    failures: List[tuple] = field(default_factory=list)

    @property
    def ok(self) -> bool:
        return not self.failures


def check_mask(ref: Routing, row_ptr, col_idx, top_p: float, k_floor: int,
               rows=None) -> MaskReport:
    """Compare a candidate CSR (row order (batch, head, q-block)) with the oracle routing."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    col_idx = np.asarray(col_idx, dtype=np.int64)
    b, h, n, _ = ref.scores.shape
    flat_s = ref.scores.reshape(b * h * n, n)
    rep = MaskReport()
    rows = range(b * h * n) if rows is None else rows
    for r in rows:
        cand = col_idx[row_ptr[r]:row_ptr[r + 1]]
        res = check_row(flat_s[r], ref.rows[r], top_p, k_floor, cand)
        rep.rows += 1
        if res == "exact":
            rep.exact += 1
        elif res == "tie":
            rep.tie += 1
        elif res == "count":
            rep.count += 1
        else:
            rep.failures.append((r, res))
    return rep


@dataclass
class OutReport:
    max_abs: float
    mean_abs: float
    count: int

    def ok(self, max_tol=2e-2, mean_tol=2e-3) -> bool:
        return self.max_abs <= max_tol and self.mean_abs <= mean_tol


def compare_out(got, ref) -> OutReport:
    """Max/mean absolute difference over the entries where `ref` is defined (not NaN)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    d = np.abs(got[m] - ref[m])
    if d.size == 0:
        return OutReport(0.0, 0.0, 0)
    return OutReport(float(d.max()), float(d.mean()), int(d.size))
