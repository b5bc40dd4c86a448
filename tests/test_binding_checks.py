"""CPU tests of the binding's argument checks: the C ABI sees only pointers, so every output
and scale buffer a caller passes must have exactly the shape the call writes, or the binding
raises ValueError before anything reaches the library.

The tensors here are CPU tensors that report themselves as GPU tensors (and refuse to hand out
a pointer), so the checks run without a GPU and no call can reach the device."""
import pytest
import torch

import block_sparse_attention_gather_amd as bsa


class FakeGpu(torch.Tensor):
    @property
    def is_cuda(self):
        return True

    def data_ptr(self):
        raise AssertionError("the binding reached a device call")


def fake(shape, dtype):
    return torch.zeros(shape, dtype=dtype).as_subclass(FakeGpu)


GRID = bsa.Grid(2, 16, 16, (4, 4, 8), 128)          # N 512, n_blk 4, Npad 512
B, H, D = 1, 2, 128
NP, NB = GRID.Npad, GRID.n_blk
ROWS = B * H * NB


def attn_args():
    bf = torch.bfloat16
    return dict(q_t=fake((B, H, NP, D), bf), k_t=fake((B, H, NP, D), bf),
                v_t=fake((B, H, NP, D), bf), row_ptr=fake((ROWS + 1,), torch.int32),
                col_idx=fake((ROWS * NB,), torch.int32), grid=GRID)


@pytest.mark.parametrize("name,shape,dtype", [
    ("out", (B, H, NP - 1, D), torch.bfloat16),
    ("out", (B, H, NP, D), torch.float32),
    ("lse", (B, H, NP - 128), torch.float32),
    ("lse", (B, H, NP), torch.bfloat16),
])
def test_sparse_attn_fwd_rejects_wrong_outputs(name, shape, dtype):
    kw = attn_args()
    kw["out"] = fake((B, H, NP, D), torch.bfloat16)
    kw["lse"] = fake((B, H, NP), torch.float32)
    kw[name] = fake(shape, dtype)
    with pytest.raises(ValueError, match=name):
        bsa.sparse_attn_fwd(**kw)


def test_sparse_attn_fwd_rejects_bad_col_idx():
    kw = attn_args()
    kw["col_idx"] = fake((ROWS, NB), torch.int32)
    with pytest.raises(ValueError, match="col_idx"):
        bsa.sparse_attn_fwd(**kw)


def fp8_args():
    u8, f32 = torch.uint8, torch.float32
    return dict(q8=fake((B, H, NP, D), u8), q_scale=fake((B, H, NB), f32),
                k8=fake((B, H, NP, D), u8), k_scale=fake((B, H, NB), f32),
                v8=fake((B, H, NB, D, 128), u8), v_scale=fake((B, H), f32),
                row_ptr=fake((ROWS + 1,), torch.int32), col_idx=fake((ROWS * NB,), torch.int32),
                grid=GRID, out=fake((B, H, NP, D), torch.bfloat16), lse=fake((B, H, NP), f32))


@pytest.mark.parametrize("name,shape", [
    ("q_scale", (B, H, NB - 1)), ("k_scale", (B, H)), ("v_scale", (B, H, NB)),
    ("out", (B, H, NP, D - 8)), ("lse", (B, H, 1)),
])
def test_sparse_attn_fwd_fp8_rejects_wrong_buffers(name, shape):
    kw = fp8_args()
    kw[name] = fake(shape, kw[name].dtype)
    with pytest.raises(ValueError, match=name):
        bsa.sparse_attn_fwd_fp8(**kw)


@pytest.mark.parametrize("name,shape", [("x8", (B, H, NP - 1, D)), ("x8_scales", (B, H))])
def test_reorder_pool_fp8_rejects_wrong_outputs(name, shape):
    x = fake((B, GRID.N, H, D), torch.bfloat16)
    kw = dict(out=fake((B, H, NP, D), torch.bfloat16),
              pooled=fake((B, H, NB, D), torch.float64),
              x8=fake((B, H, NP, D), torch.uint8), x8_scales=fake((B, H, NB), torch.float32))
    kw[name] = fake(shape, kw[name].dtype)
    with pytest.raises(ValueError, match=name):
        bsa.reorder_pool(x, GRID, fp8=True, **kw)


@pytest.mark.parametrize("name,shape", [("out", (B, H, NP, 64)), ("v8", (B, H, NB, D, 64)),
                                        ("v_scales", (H,))])
def test_reorder_quantize_v_rejects_wrong_outputs(name, shape):
    x = fake((B, GRID.N, H, D), torch.bfloat16)
    kw = dict(out=fake((B, H, NP, D), torch.bfloat16), v8=fake((B, H, NB, D, 128), torch.uint8),
              v_scales=fake((B, H), torch.float32))
    kw[name] = fake(shape, kw[name].dtype)
    with pytest.raises(ValueError, match=name):
        bsa.reorder_quantize_v(x, GRID, **kw)
