"""Test-side pieces of the FP8 parity tests.

1. The byte layout of the FP8 V codes the library writes (bsa_quantize_fp8 with v_layout = 1,
bsa_reorder_quantize_v), as its header documents it, and the map to the token-major layout in
which the oracle quantizes V (the oracle itself knows nothing of the library's layouts).

Every block of B keys is stored transposed, [feature][key position], and key position
64c + 32h + b (c = 64-key chunk, h = half, b = byte in the half) holds key
64c + 32(b / 16) + 8((b % 16) / 4) + 4h + b % 4 of the block.

2. The per-element output tolerance of the FP8 attention against the oracle's exact fp64
attention over the dequantized inputs (fp8_out_tol).
"""
import numpy as np


def v8_key_order(B: int) -> np.ndarray:
    """Key of the block held at each key position of a transposed V row."""
    pos = np.arange(B)
    c, h, b = pos // 64, (pos % 64) // 32, pos % 32
    return 64 * c + 32 * (b // 16) + 8 * ((b % 16) // 4) + 4 * h + b % 4


def v8_to_tokens(v8: np.ndarray) -> np.ndarray:
    """[b, h, n_blk, D, B] block-transposed codes -> [b, h, n_blk * B, D] token-major codes."""
    bb, hh, n, D, B = v8.shape
    out = np.empty((bb, hh, n, B, D), v8.dtype)
    out[:, :, :, v8_key_order(B), :] = np.swapaxes(v8, 3, 4)
    return out.reshape(bb, hh, n * B, D)


def tokens_to_v8(codes: np.ndarray, B: int) -> np.ndarray:
    """[b, h, Npad, D] token-major codes -> [b, h, n_blk, D, B] block-transposed codes."""
    bb, hh, Np, D = codes.shape
    blocks = codes.reshape(bb, hh, Np // B, B, D)
    return np.ascontiguousarray(np.swapaxes(blocks[:, :, :, v8_key_order(B), :], 3, 4))


# Rounding of the kernel's own fp32 arithmetic, relative to sum_u w_u |v_u|:
#  * logits: products of E4M3 codes are exact in fp32; two fp32 roundings per 64-term MFMA step
#    over D = 128 and the fp32 product of the scales leave each logit within
#    2^-22 * scale * sum_d |q_d k_d| of its exact value, below 2^-16 for these workloads
#    (scale * sum_d |q_d k_d| < 64), so a weight moves by a factor within 1 +- 2^-15;
#  * exp2 and the running-max subtraction: a few fp32 ulps (2^-21);
#  * the fp32 accumulation of P V and of the row sum over at most 2^11 MFMA steps (2^17 keys):
#    within 2^11 * 2^-24 = 2^-13; the final division: one ulp.
# 2^-10 covers their sum (about 2^-12.5) with room to spare.
FP32_ARITH_REL = 2.0 ** -10
# bf16 output: round to nearest even with an 8-bit significand, |fl(x) - x| <= 2^-8 |x|.
BF16_OUT_REL = 2.0 ** -8


def fp8_out_tol(cast_bound, ref, wabs):
    """Largest |O_gpu - O_ref| allowed per element, with O_ref the exact fp64 attention over the
    dequantized inputs:
      cast_bound   what casting the probabilities to E4M3 can change (the oracle's
                   attn_error_bound or expcast_error_bound);
      wabs         sum_u w_u |v_u| (the oracle's abs_weighted_v), times FP32_ARITH_REL for
                   the kernel's fp32 arithmetic;
      ref          |O_ref|: the bf16 output rounding is at most 2^-8 |O_gpu|, and
                   |O_gpu| <= |O_ref| + cast_bound + fp32 term.
    """
    e = cast_bound + FP32_ARITH_REL * wabs
    return e + BF16_OUT_REL * (np.abs(ref) + e)
