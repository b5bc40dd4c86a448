"""Pin of the oracle's bf16 -> fp64 widening (every bf16 input of the oracle passes through
it): on all 65,536 bit patterns it gives PyTorch's own bfloat16 -> float64 conversion, bit for
bit (signed zeros, subnormals, infinities), and NaN exactly where PyTorch gives NaN."""
import numpy as np
import torch

from oracle import widen_bf16


def test_widen_bf16_all_patterns_match_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):             # signalling NaN patterns are quietened
        got = widen_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert got.dtype == np.float64 and got.shape == (1 << 16,)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127                      # exponent all ones, mantissa non-zero
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))


def test_widen_bf16_known_values():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x0001 = smallest subnormal 2^-133, 0x7F7F = largest finite
    got = widen_bf16(np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x8000], np.uint16))
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 2.0 ** -133
    assert got[3] == (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert got[4] == 0.0 and np.signbit(got[4])
