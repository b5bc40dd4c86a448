"""GPU check that the attention results do not depend on the schedule.

A layer large enough that pairs of XCDs share a queue (eight heads' K and V past the 256 MiB
MALL, in bf16 and in E4M3: 16 heads of 134,400 tokens) must give, head by head and bit for bit,
the output and LSE of the same head run alone (one head: the few-heads mode, one queue that
every workgroup takes from).  Every row keeps at most seven key blocks, fewer than the smallest
chunk, so no row is split under either schedule and each row is computed by one work item in
both runs.  Covers the bf16 kernel and the FP8 kernel with both casts.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_gather_amd as bsa

from plan_ref import queue_group

pytestmark = pytest.mark.gpu

HEADS = 16
GRID = bsa.Grid(42, 40, 80, (4, 4, 8), 128)          # 134,400 tokens, 1050 blocks a row


def _csr(heads, n):
    """Row i of head h: blocks i-1 .. i+1 and the first h mod 4 blocks (at most 7)."""
    cols = []
    for hh in range(heads):
        for i in range(n):
            cols.append(np.union1d(np.arange(max(0, i - 1), min(n, i + 2)), np.arange(hh % 4)))
    rp = np.concatenate([[0], np.cumsum([len(c) for c in cols])]).astype(np.int32)
    return rp, np.concatenate(cols).astype(np.int32)


def _head_csr(rp, ci, hh, n):
    lo, hi = int(rp[hh * n]), int(rp[(hh + 1) * n])
    return (torch.from_numpy(rp[hh * n:(hh + 1) * n + 1] - lo).to("cuda:0"),
            torch.from_numpy(ci[lo:hi].copy()).to("cuda:0"))


@pytest.fixture(scope="module")
def layer():
    n = GRID.n_blk
    assert queue_group(4 * GRID.Npad * 128) == 2          # bf16 K and V: pairs
    assert queue_group(2 * GRID.Npad * 128) == 2          # E4M3 K and V: pairs too
    gen = torch.Generator(device="cuda:0").manual_seed(7)
    q, k, v = (torch.randn((1, HEADS, GRID.Npad, 128), generator=gen, device="cuda:0")
               .to(torch.bfloat16) for _ in range(3))
    rp, ci = _csr(HEADS, n)
    print(f"[gpu] schedule test layer: heads {HEADS} n_blk {n} nnz {int(rp[-1])}", flush=True)
    return q, k, v, rp, ci


def test_bf16_pairs_equal_single_heads(layer):
    q, k, v, rp, ci = layer
    n = GRID.n_blk
    ws = torch.zeros(bsa.attn_workspace_bytes(1, HEADS, 128, GRID), dtype=torch.uint8,
                     device="cuda:0")
    out, lse = bsa.sparse_attn_fwd(q, k, v, torch.from_numpy(rp).to("cuda:0"),
                                   torch.from_numpy(ci).to("cuda:0"), GRID, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[4:8].cpu().view(torch.int32)[0]) == 2    # header word 1: XCDs per queue
    for hh in range(HEADS):
        rph, cih = _head_csr(rp, ci, hh, n)
        o1, l1 = bsa.sparse_attn_fwd(q[:, hh:hh + 1].contiguous(), k[:, hh:hh + 1].contiguous(),
                                     v[:, hh:hh + 1].contiguous(), rph, cih, GRID)
        torch.cuda.synchronize()
        assert torch.equal(o1, out[:, hh:hh + 1]), hh
        assert torch.equal(l1.view(torch.int32), lse[:, hh:hh + 1].view(torch.int32)), hh
    print("[gpu]   bf16: 16 heads under queue pairs = each head alone, bit for bit", flush=True)


@pytest.mark.parametrize("expcast", [False, True], ids=["rne", "expcast"])
def test_fp8_pairs_equal_single_heads(layer, expcast):
    q, k, v, rp, ci = layer
    n = GRID.n_blk
    q8, qs = bsa.quantize_fp8(q, GRID)
    k8, ks = bsa.quantize_fp8(k, GRID)
    v8, vs = bsa.quantize_fp8(v, GRID, v_layout=True)
    out, lse = bsa.sparse_attn_fwd_fp8(q8, qs, k8, ks, v8, vs, torch.from_numpy(rp).to("cuda:0"),
                                       torch.from_numpy(ci).to("cuda:0"), GRID, expcast=expcast)
    torch.cuda.synchronize()
    for hh in range(HEADS):
        rph, cih = _head_csr(rp, ci, hh, n)
        s = slice(hh, hh + 1)
        o1, l1 = bsa.sparse_attn_fwd_fp8(
            q8[:, s].contiguous(), qs[:, s].contiguous(), k8[:, s].contiguous(),
            ks[:, s].contiguous(), v8[:, s].contiguous(), vs[:, s].contiguous(), rph, cih, GRID,
            expcast=expcast)
        torch.cuda.synchronize()
        assert torch.equal(o1, out[:, s]), hh
        assert torch.equal(l1.view(torch.int32), lse[:, s].view(torch.int32)), hh
    print(f"[gpu]   fp8 expcast={expcast}: 16 heads under queue pairs = each head alone",
          flush=True)
