"""GPU check of the device planner: after bsa_sparse_attn_fwd the caller-owned workspace holds
the schedule the planner kernels built; it must equal, word for word, the schedule of the
library's sequential host planner (plan_host.h, compiled for the CPU by tests/plan_ref.py) on
the same CSR: chunk size, queue starts and lengths, every work item, partial-slot bases.
Cases: routed masks, every row dense (split rows), one dense head among sparse ones; 6 heads
(few-heads mode, one queue) and 20 heads (head mode, XCD queues); and heads long enough that
pairs of XCDs share a queue (Wan-2.1-720p's grid: eight heads' bf16 K and V exceed the MALL)."""

import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa
from workloads import Config, gen_qkv

from gpu_common import grid_of, to_dev
from plan_ref import KNQ, layout, plan, queue_group

pytestmark = pytest.mark.gpu


def _slots_of(ws_bytes, bh, n_blk, B, D):
    for s in range(1, 1 << 14):
        if layout(bh, n_blk, B, D, s)["total"] == ws_bytes:
            return s
    raise AssertionError("workspace size matches no slot count")


def _device_plan(cfg, rp, ci, q_t, k_t, v_t, grid):
    h, D, B = cfg.heads, cfg.head_dim, cfg.block
    n = grid.n_blk
    ws_bytes = bsa.attn_workspace_bytes(1, h, D, grid)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda:0")
    bsa.sparse_attn_fwd(q_t, k_t, v_t, rp, ci, grid, workspace=ws)
    torch.cuda.synchronize()
    slots = _slots_of(ws_bytes, h, n, B, D)
    L = layout(h, n, B, D, slots)
    w = ws.cpu().numpy()
    hdr = w[L["hdr"]:L["hdr"] + 4 * (32 + 33 * KNQ)].view(np.int32)
    qstart = hdr[8:8 + KNQ]
    qlen = hdr[32 + 32 * KNQ:32 + 33 * KNQ]
    nit = int(qlen.sum())
    items = w[L["items"]:L["items"] + 16 * nit].view(np.int32).reshape(nit, 4)
    sbase = w[L["head_slot_base"]:L["head_slot_base"] + 4 * h].view(np.int32)
    return dict(Kc=int(hdr[0]), group=int(hdr[1]), qstart=qstart, qlen=qlen, items=items,
                slot_base=sbase, slots=slots)


@pytest.mark.parametrize("heads", [6, 20], ids=["few_heads_mode", "head_mode"])
@pytest.mark.parametrize("case", ["routed", "dense", "one_dense_head"])
def test_device_plan_equals_host_plan(case, heads):
    cfg = Config("gplan", 6, 20, 40, heads, 128, 128, (4, 4, 8), 0.85, 4, 151)
    q, k, v = gen_qkv(cfg, gains=np.linspace(0.6, 2.0, cfg.heads))
    grid = grid_of(cfg)
    q_t, k_t, v_t = (bsa.reorder(to_dev(x), grid) for x in (q, k, v))
    n, h = grid.n_blk, cfg.heads
    if case == "routed":
        rp, ci, _ = bsa.score_and_route(q_t, k_t, grid, cfg.top_p, cfg.k_floor)
    else:
        dense = np.ones((h, n, n), bool) if case == "dense" else np.eye(n, dtype=bool)[None].repeat(h, 0)
        if case == "one_dense_head":
            dense[2] = True
        cols = [np.nonzero(dense[hh, i])[0] for hh in range(h) for i in range(n)]
        rp_h = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
        rp = torch.from_numpy(rp_h).to("cuda:0")
        ci = torch.from_numpy(np.concatenate(cols).astype(np.int32)).to("cuda:0")
    torch.cuda.synchronize()
    print(f"[gpu] device plan {case}: heads {h} n_blk {n} nnz {int(rp[-1].item())}", flush=True)
    got = _device_plan(cfg, rp, ci, q_t, k_t, v_t, grid)
    group = queue_group(4 * grid.Npad * cfg.head_dim) if heads >= 16 else 1
    assert got["group"] == group == 1
    want = plan(rp.cpu().numpy(), n, h, 2 * got["slots"], group)
    assert got["Kc"] == want["Kc"]
    assert np.array_equal(got["qstart"], want["qstart"])
    assert np.array_equal(got["qlen"], want["qlen"])
    assert np.array_equal(got["items"], want["items"])
    if heads >= 16:                  # the few-heads mode numbers partial slots in item order
        assert np.array_equal(got["slot_base"], want["slot_base"])
    print(f"[gpu]   {len(want['items'])} items, Kc {want['Kc']}, identical", flush=True)


def test_device_plan_queue_pairs():
    """16 heads on Wan-2.1-720p's grid (75,648 padded tokens, 37 MiB of bf16 K and V a head):
    the planner lets pairs of XCDs share queues 0, 2, 4 and 6, and writes the host planner's
    schedule for that grouping word for word.  Random Q, K, V on the device; each head keeps a
    band of blocks around the diagonal, wider for some heads, plus the first block."""
    cfg = Config("gpairs", 21, 45, 80, 16, 128, 128, (4, 4, 8), 0.85, 8, 152)
    grid = grid_of(cfg)
    n, h = grid.n_blk, cfg.heads
    gen = torch.Generator(device="cuda:0").manual_seed(152)
    q_t, k_t, v_t = (torch.randn((1, h, grid.Npad, 128), generator=gen, device="cuda:0")
                     .to(torch.bfloat16) for _ in range(3))
    cols = []
    for hh in range(h):
        w = 1 + hh % 4
        for i in range(n):
            cols.append(np.union1d([0], np.arange(max(0, i - w), min(n, i + w + 1))))
    rp_h = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    rp = torch.from_numpy(rp_h).to("cuda:0")
    ci = torch.from_numpy(np.concatenate(cols).astype(np.int32)).to("cuda:0")
    torch.cuda.synchronize()
    print(f"[gpu] device plan, queue pairs: heads {h} n_blk {n} nnz {int(rp_h[-1])}", flush=True)
    got = _device_plan(cfg, rp, ci, q_t, k_t, v_t, grid)
    group = queue_group(4 * grid.Npad * 128)
    assert got["group"] == group == 2
    want = plan(rp_h, n, h, 2 * got["slots"], group)
    assert got["Kc"] == want["Kc"]
    assert np.array_equal(got["qstart"], want["qstart"])
    assert np.array_equal(got["qlen"], want["qlen"])
    assert (got["qlen"][0::2] > 0).all() and not got["qlen"][1::2].any()
    assert np.array_equal(got["items"], want["items"])
    assert np.array_equal(got["slot_base"], want["slot_base"])
    print(f"[gpu]   {len(want['items'])} items, Kc {want['Kc']}, identical", flush=True)
