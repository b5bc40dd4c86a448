"""CPU tests of the attention schedule (the library's sequential host planner, plan_host.h, on
the arithmetic the planner kernels share, plan.h): on ordinary and pathologically skewed row
lengths, every (row, key block) pair lands in exactly one work item, split rows respect the
chunk bound and the workspace bounds, the queue layout follows its definition (head mode: heads
longest-first to the least-loaded XCD queue, or to every other queue when pairs of XCDs share
one; few-heads mode: one queue in global cost order), and the output is deterministic.  A GPU test checks that the device planner writes this same
schedule."""
import numpy as np
import pytest

from plan_ref import KNQ, plan, queue_group

pytestmark = pytest.mark.slow


def _row_ptr(costs):
    return np.concatenate([[0], np.cumsum(costs)]).astype(np.int32)


def check(costs, n_blk, nbh, target, group=1):
    costs = np.asarray(costs, np.int64).reshape(nbh * n_blk)
    rp = _row_ptr(costs)
    P = plan(rp, n_blk, nbh, target, group)
    nnz = int(costs.sum())
    Kc = max(8, -(-nnz // target))
    assert P["Kc"] == Kc
    it = P["items"]
    rows = nbh * n_blk
    assert len(it) <= rows + target                          # workspace bound on items
    # items of every row: its CSR range split into consecutive chunks of at most Kc blocks
    order = np.lexsort((it[:, 1], it[:, 0]))
    by_row = it[order]
    starts = np.searchsorted(by_row[:, 0], np.arange(rows + 1))
    used_slots = np.zeros(2 * target, bool)
    for r in range(rows):
        sub = by_row[starts[r]:starts[r + 1]]
        c = int(costs[r])
        ni = max(1, -(-c // Kc))
        assert len(sub) == ni, (r, c, len(sub), ni)
        assert sub[0, 1] == rp[r] and sub[-1, 2] == rp[r + 1]
        assert np.all(sub[1:, 1] == sub[:-1, 2])               # no gap, no overlap
        assert np.all(sub[:, 2] - sub[:, 1] <= Kc)
        if c > 0:
            assert np.all(sub[:, 2] > sub[:, 1])
        if ni == 1:
            assert sub[0, 3] == -1
        else:
            s0 = sub[0, 3]
            assert np.all(sub[:, 3] == s0) and 0 <= s0 and s0 + ni <= 2 * target
            assert not used_slots[s0:s0 + ni].any()
            used_slots[s0:s0 + ni] = True
    # heads ranked by cost descending, ties by index
    hc = costs.reshape(nbh, n_blk).sum(axis=1)
    want_rank = np.empty(nbh, np.int64)
    want_rank[sorted(range(nbh), key=lambda h: (-hc[h], h))] = np.arange(nbh)
    assert np.array_equal(P["head_rank"], want_rank)
    # partial-slot bases (head mode): split chunks per head, heads in index order
    split = np.where(costs > Kc, -(-costs // Kc), 0).reshape(nbh, n_blk).sum(axis=1)
    if not (nbh < 16 and nbh * n_blk <= 16384):
        assert np.array_equal(P["slot_base"], np.concatenate([[0], np.cumsum(split)[:-1]]))
    # queues
    assert np.array_equal(P["qstart"], np.concatenate([[0], np.cumsum(P["qlen"])[:-1]]))
    assert P["qlen"].sum() == len(it)
    rws = it[:, 0]
    first = np.concatenate([[True], rws[1:] != rws[:-1]])
    seq = rws[first]                                          # rows in item order
    assert len(np.unique(seq)) == len(seq)                    # a row's chunks are adjacent
    if nbh < 16 and nbh * n_blk <= 16384:
        # few-heads mode: one queue, all rows by cost descending, ties by row
        assert P["qlen"][0] == len(it) and not P["qlen"][1:].any()
        keyv = [(-int(costs[x]), int(x)) for x in seq]
        assert keyv == sorted(keyv)
    else:
        # head mode: heads longest first to the least-loaded queue in use (every group-th,
        # ties: lowest); in a queue the heads in rank order, each head's rows by cost
        # descending (ties by row)
        used = np.arange(0, KNQ, group)
        assert not np.delete(P["qlen"], used).any()
        qload = np.zeros(KNQ, np.int64)
        hq = np.zeros(nbh, np.int64)
        for h in sorted(range(nbh), key=lambda x: (-hc[x], x)):
            q = int(used[np.argmin(qload[used])])
            qload[q] += hc[h]
            hq[h] = q
        head = it[:, 0] // n_blk
        for q in range(KNQ):
            seg = slice(P["qstart"][q], P["qstart"][q] + P["qlen"][q])
            assert np.all(hq[head[seg]] == q)
            assert np.all(np.diff(P["head_rank"][head[seg]]) >= 0)
        hs = seq // n_blk
        for hh in range(nbh):
            sub = seq[hs == hh]
            keyv = [(-int(costs[x]), int(x)) for x in sub]
            assert keyv == sorted(keyv)
    # deterministic
    P2 = plan(rp, n_blk, nbh, target, group)
    assert all(np.array_equal(P[k], P2[k]) for k in P if k != "Kc")
    return P, costs


def _queue_rho(P, costs, n_blk, group=1):
    it = P["items"]
    loads = [int((it[s:s + n, 2] - it[s:s + n, 1]).sum())
             for s, n in zip(P["qstart"][::group], P["qlen"][::group])]
    return max(loads) / np.mean(loads)


def test_uniform_heads():
    rng = np.random.default_rng(0)
    check(rng.integers(8, 120, size=40 * 256), 256, 40, 1024)


def test_one_dense_head_among_sparse_ones():
    n = 300
    costs = np.ones((24, n), np.int64)
    costs[5] = n                                                # every row of head 5 is dense
    P, c = check(costs, n, 24, 1024)
    # the dense head fills one queue on its own; the others share the rest
    it = P["items"]
    q5 = [q for q in range(KNQ) if np.any(it[P["qstart"][q]:P["qstart"][q] + P["qlen"][q], 0]
                                          // n == 5)][0]
    heads_q5 = np.unique(it[P["qstart"][q5]:P["qstart"][q5] + P["qlen"][q5], 0] // n)
    assert list(heads_q5) == [5]


def test_one_huge_row_is_split():
    n = 4096
    costs = np.zeros((2, n), np.int64)
    costs[1, 17] = n                                            # one dense row, the rest empty
    costs[0, :10] = 3
    P, _ = check(costs, n, 2, 64)
    assert P["Kc"] == -(-(n + 30) // 64)                        # 65
    assert (P["items"][:, 0] == n + 17).sum() == -(-n // P["Kc"])


def test_all_rows_dense_many_splits():
    n = 96
    P, _ = check(np.full(3 * n, n), n, 3, 64)                  # Kc = 432 -> no split
    P, _ = check(np.full(3 * n, n), n, 3, 4096)                # Kc = 8 -> 12 chunks a row
    assert P["Kc"] == 8 and len(P["items"]) == 3 * n * 12


@pytest.mark.parametrize("heads", [1, 3, 5])
def test_few_heavy_skewed_heads(heads):
    rng = np.random.default_rng(heads)
    n = 591
    dens = rng.uniform(0.1, 0.7, size=heads)
    costs = np.stack([rng.binomial(n, d, size=n) + 1 for d in dens])
    P, c = check(costs, n, heads, 1024)
    assert P["qlen"][0] == len(P["items"])                     # few-heads mode: one queue


@pytest.mark.parametrize("n_blk", [1, 2, 7, 9])
def test_tiny_heads_leave_slabs_empty(n_blk):
    rng = np.random.default_rng(n_blk)
    check(rng.integers(0, n_blk + 1, size=5 * n_blk), n_blk, 5, 32)


def test_many_heads():
    rng = np.random.default_rng(7)
    P, c = check(rng.integers(1, 4, size=2048 * 4), 4, 2048, 1024)
    assert _queue_rho(P, c, 4) < 1.01                           # LPT over 2048 small heads


def test_wan720p_like_heterogeneous_heads():
    """40 heads whose densities spread from 10 % to 70 % (the shape of the load-balancer
    stress layer): LPT over whole heads keeps the eight XCD queues within 5 % of each other
    (the rest is left to the workgroups that steal from other queues once their own is
    empty)."""
    rng = np.random.default_rng(11)
    n = 591
    dens = rng.permutation(np.linspace(0.1, 0.7, 40))
    costs = np.stack([np.clip(rng.binomial(n, d, size=n), 8, n) for d in dens])
    P, c = check(costs, n, 40, 1024)
    assert _queue_rho(P, c, n) < 1.05


def test_mode_boundary():
    rng = np.random.default_rng(12)
    P, _ = check(rng.integers(1, 20, size=15 * 64), 64, 15, 512)    # 15 heads: one queue
    assert P["qlen"][0] == len(P["items"])
    P, _ = check(rng.integers(1, 20, size=16 * 64), 64, 16, 512)    # 16 heads: XCD queues
    assert (P["qlen"] > 0).sum() == KNQ
    P, _ = check(rng.integers(1, 20, size=5 * 4096), 4096, 5, 512)  # 20480 rows: XCD queues
    assert (P["qlen"] > 0).sum() == 5


def test_rows_without_blocks_are_single_empty_items():
    costs = np.zeros(4 * 16, np.int64)
    costs[::5] = 9
    P, _ = check(costs, 16, 4, 16)
    it = P["items"]
    assert np.sum(it[:, 2] == it[:, 1]) == np.sum(costs == 0)


def test_queue_groups_rule():
    """Pairs of XCDs share a queue once eight heads' K and V (one head a queue) exceed the
    256 MiB MALL: the bf16 HunyuanVideo-720p and Wan-2.1-720p layers (58 and 37 MiB a head),
    not Wan-2.1-480p (16 MiB) nor the E4M3 copy of HunyuanVideo-720p (29 MiB)."""
    kv = lambda n_blk, elem: 2 * n_blk * 128 * 128 * elem
    assert queue_group(kv(929, 2)) == 2                 # HunyuanVideo-720p, bf16
    assert queue_group(kv(929, 1)) == 1                 # the same, E4M3
    assert queue_group(kv(591, 2)) == 2                 # Wan-2.1-720p
    assert queue_group(kv(256, 2)) == 1                 # Wan-2.1-480p
    assert queue_group(32 << 20) == 1 and queue_group((32 << 20) + 1) == 2


@pytest.mark.parametrize("heads", [16, 24, 40])
def test_queue_pairs(heads):
    """Pairs sharing a queue: the heads go longest-first to queues 0, 2, 4 and 6 only, which
    stay within 5 % of each other; the odd queues are empty."""
    rng = np.random.default_rng(heads)
    n = 929
    dens = rng.permutation(np.linspace(0.2, 0.6, heads))
    costs = np.stack([np.clip(rng.binomial(n, d, size=n), 8, n) for d in dens])
    P, c = check(costs, n, heads, 1024, group=2)
    assert (P["qlen"][0::2] > 0).all() and not P["qlen"][1::2].any()
    assert _queue_rho(P, c, n, group=2) < 1.05
