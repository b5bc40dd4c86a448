"""FP8 (e4m3) attention, oracle side.

TEST INFRASTRUCTURE ONLY: imported by the tests and the bench's CPU leg, never by the product
path; shares no code with the HIP kernels.

Source: VC-Attention page ("VC-Attention: Value Smoothing and Softmax Casting for Low-bit
Attention", abstract): a low-bit attention kernel whose two matrix products run on low-bit
tensor cores, quantized per hardware block with a scale set by the block's largest entry, and
whose probabilities are cast to E4M3 codes between the exponential and the second product.
Readings used here:

* E4M3 is the OCP 8-bit format with 4 exponent bits (bias 7), 3 mantissa bits, subnormals,
  largest finite value 448 and no infinities; conversion rounds to nearest, ties to even.
* Q and K are quantized per block of B tokens of one (batch, head): s = amax / 448 over the
  block's B x D values, code = e4m3(x * (448 / amax)) in fp32 (a block of zeros: s = 0,
  codes 0).  V is quantized with one scale per (batch, head) (amax over all its tokens), so
  the second product needs no per-block rescaling.
* The probabilities of one query row are exp(l_u - m) for the logits l_u = scale * <q, k_u>
  of the dequantized Q and K, m the running maximum over the key blocks taken so far in the
  row's column order, multiplied by 2^8 and cast to E4M3 (so the largest is 256, inside the
  format's normal range); the row sum is kept unquantized.  The output is
  (sum_u P8_u v_u) / (sum_u p_u) for the dequantized v_u.

`e4m3_round` is written from the format definition and pinned against PyTorch's
float8_e4m3fn conversion.  `attn_error_bound` bounds what casting the probabilities to E4M3
alone can change in the output (derived below); the tests compare the GPU's FP8 attention
with the exact fp64 attention over the dequantized inputs against that bound.
"""
from __future__ import annotations

import numpy as np

from .bsa_oracle import num_blocks, widen_bf16

E4M3_MAX = 448.0
P_OFFSET_LOG2 = 8          # probabilities are cast as 2^8 * exp(l - m)


def e4m3_round(x) -> np.ndarray:
    """fp32 values -> E4M3 codes (uint8), round to nearest even; |x| <= 448 expected."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)     # exact widening
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    if np.any(a > 464.0):                                       # 464 rounds past 448
        raise ValueError("value outside the E4M3 range")
    codes = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    # subnormals: multiples of 2^-9
    q = np.rint(a[sub] * 2.0 ** 9)                              # rint: ties to even
    codes[sub] = q.astype(np.uint8)                             # q == 8 is the smallest normal
    # normals: exponent e in [-6, 8], 3 mantissa bits
    an = a[~sub]
    e = np.floor(np.log2(an)).astype(np.int64)
    frac = an / np.exp2(e) - 1.0                                # [0, 1)
    mq = np.rint(frac * 8.0)
    carry = mq >= 8
    e = e + carry
    mq = np.where(carry, 0, mq)
    codes[~sub] = ((e + 7) << 3 | mq.astype(np.int64)).astype(np.uint8)
    return codes | sign


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    v = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7))
    if np.any((e == 0xF) & (m == 0x7)):
        raise ValueError("NaN code")
    return s * v


def _scale_codes(x32, amax):
    """codes of x32 (fp32) with the scale set by amax (fp32); returns (codes, s)."""
    amax = np.float32(amax)
    if amax == 0:
        return np.zeros(x32.shape, np.uint8), np.float32(0.0)
    inv = np.float32(np.float32(E4M3_MAX) / amax)
    return e4m3_round(x32 * inv), np.float32(amax / np.float32(E4M3_MAX))


def quantize_rows(xt_bits, B: int):
    """Per-block E4M3 of tiled bf16 [b, h, Npad, D] -> (codes [b, h, Npad, D] u8,
    scales [b, h, n_blk] f32)."""
    x = widen_bf16(xt_bits).astype(np.float32)                  # exact
    b, h, Np, D = x.shape
    n = Np // B
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty((b, h, n), np.float32)
    for bi in range(b):
        for hi in range(h):
            for j in range(n):
                blk = x[bi, hi, j * B:(j + 1) * B]
                codes[bi, hi, j * B:(j + 1) * B], scales[bi, hi, j] = _scale_codes(
                    blk, np.abs(blk).max())
    return codes, scales


def quantize_v(vt_bits, B: int):
    """Per-(batch, head) E4M3 of tiled bf16 V [b, h, Npad, D] -> (codes [b, h, Npad, D] u8
    in the same token-major layout, scales [b, h] f32): one scale set by the largest entry of
    the whole (batch, head), so the second product needs no per-block rescaling."""
    x = widen_bf16(vt_bits).astype(np.float32)
    b, h, Np, D = x.shape
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty((b, h), np.float32)
    for bi in range(b):
        for hi in range(h):
            codes[bi, hi], scales[bi, hi] = _scale_codes(x[bi, hi], np.abs(x[bi, hi]).max())
    return codes, scales


def dequantize_rows(codes, scales, B: int) -> np.ndarray:
    """Per-block codes [b, h, Npad, D] and scales [b, h, n_blk] -> fp64 [b, h, Npad, D]."""
    v = e4m3_decode(codes)
    return v * np.repeat(scales.astype(np.float64), B, axis=2)[..., None]


def dequantize_v(codes, scales) -> np.ndarray:
    """Per-head codes [b, h, Npad, D] and scales [b, h] -> fp64 [b, h, Npad, D]."""
    return e4m3_decode(codes) * scales.astype(np.float64)[:, :, None, None]


def attn_error_bound(q, k, v, row_ptr, col_idx, N: int, B: int, scale: float, rows):
    """Per-element bound on |O_fp8 - O| for the listed rows (b, h, i) of fp64 inputs q, k, v
    [b, h, Npad, D] (the dequantized tensors) and the exact attention O over them.

    Only the probabilities are rounded: each cast value P8 = e4m3(e) of e = 2^8 exp(l - m)
    <= 256 differs from e by at most half a unit in the last place, i.e. by
    <= 2^-4 e (normal codes) or <= 2^-10 (subnormal codes, e < 2^-6).  The row sum L of the
    e's is >= 2^8 (the element that set the running maximum contributes 2^8).  So
        |dO| <= sum_u (2^-4 e_u + 2^-10) |v_u| / L <= 2^-4 sum_u w_u |v_u| + 2^-18 sum_u |v_u|
    with w_u the exact softmax weights.  Returns {row: bound [rows of the block, D]}."""
    n = num_blocks(N, B)
    out = {}
    for (bi, hi, i) in rows:
        r = (bi * q.shape[1] + hi) * n + i
        sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
        keys = np.concatenate([np.arange(j * B, min((j + 1) * B, N)) for j in sel])
        lo, hi_ = i * B, min((i + 1) * B, N)
        lg = scale * (q[bi, hi, lo:hi_] @ k[bi, hi, keys].T)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        av = np.abs(v[bi, hi, keys])
        out[(bi, hi, i)] = 2.0 ** -4 * (w @ av) + 2.0 ** -18 * av.sum(axis=0)[None, :]
    return out


def abs_weighted_v(q, k, v, row_ptr, col_idx, N: int, B: int, scale: float, rows):
    """sum_u w_u |v_u| per element for the listed rows (b, h, i): the exact softmax weights
    w of the row's real keys over fp64 q, k, v [b, h, Npad, D], applied to |v|.  It is the
    size against which rounding in the kernel's fp32 arithmetic is measured (a relative error
    r in every weight moves the output by at most r times this).  Returns
    {row: [rows of the block, D]}."""
    n = num_blocks(N, B)
    out = {}
    for (bi, hi, i) in rows:
        r = (bi * q.shape[1] + hi) * n + i
        sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
        keys = np.concatenate([np.arange(j * B, min((j + 1) * B, N)) for j in sel])
        lo, hi_ = i * B, min((i + 1) * B, N)
        lg = scale * (q[bi, hi, lo:hi_] @ k[bi, hi, keys].T)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[(bi, hi, i)] = w @ np.abs(v[bi, hi, keys])
    return out


# ---------------------------------------------------------------------------------------
# ExpCast (VC-Attention page, abstract: log-domain scores mapped straight to E4M3 codes with
# one fused multiply-add, no exponential)
# ---------------------------------------------------------------------------------------
EXPCAST_DELTA = 2.0 ** 0.1475 - 1.0      # largest relative deviation of a cast value (below)
EXPCAST_ABS = 2.0 ** -6                  # absolute deviation bound below the normal range


def expcast_codes(y, rounding: str = "nearest") -> np.ndarray:
    """Codes for log2 probabilities y (the 2^8-scaled probability is 2^y, y <= 8): the E4M3
    code of 2^y has exponent field floor(y) + 7 above 3 mantissa bits, and taking the mantissa
    linear in the fraction of y gives the code 8y + 56 (its exponent-field part is exact).
    Converted to an unsigned byte, clamped to [0, 255], by rounding to nearest (ties to even)
    or by truncation (rounding="floor")."""
    t = 8.0 * np.asarray(y, dtype=np.float64) + 56.0
    t = np.where(np.isnan(t), 0.0, t)
    r = np.rint(t) if rounding == "nearest" else np.floor(t)
    return np.clip(r, 0, 255).astype(np.uint8)


def expcast_error_bound(q, k, v, row_ptr, col_idx, N: int, B: int, scale: float, rows):
    """Per-element bounds (on |O_expcast - O| and on |lse_expcast - lse|) for the listed rows.

    For an integer code c = 8E + M taken for t = 8y + 56 with t - c = r in [-1/2, 1) (either
    rounding), the cast value 2^(E-7)(1 + M/8) differs from 2^y by log2 of
    (log2(1 + M/8) - M/8) - r/8, in [-1/8, 0.085 + 1/16]: a factor in
    [2^-0.125, 2^0.1475], so within EXPCAST_DELTA relatively.  Below 2^-6 the codes are
    subnormal (value c 2^-9) and both values lie in [0, 2^-6]: within EXPCAST_ABS.  Every
    error is then scaled by the rescale factors (<= 1) into the frame of the final maximum, where
    the probabilities are e_u = 2^8 exp(l_u - max l) with sum L >= 2^8.  The output is the
    average weighted by the cast values P8_u = e_u + eps_u and normalized by their own sum
    (L + sum eps), so
        |dO| <= [sum |eps_u| |v_u| + (sum |eps_u|) sum w_u |v_u|] / (L - sum |eps_u|)
    with |eps_u| <= DELTA e_u + ABS and w_u = e_u / L, and |dlse| <= max(-ln(1 - E), ln(1 + E))
    for E = sum |eps| / L.  Returns {row: (bound on O [rows, D], bound on lse [rows])}."""
    n = num_blocks(N, B)
    d, A = EXPCAST_DELTA, EXPCAST_ABS
    out = {}
    for (bi, hi, i) in rows:
        r = (bi * q.shape[1] + hi) * n + i
        sel = col_idx[row_ptr[r]:row_ptr[r + 1]]
        keys = np.concatenate([np.arange(j * B, min((j + 1) * B, N)) for j in sel])
        lo, hi_ = i * B, min((i + 1) * B, N)
        lg = scale * (q[bi, hi, lo:hi_] @ k[bi, hi, keys].T)
        e = 2.0 ** 8 * np.exp(lg - lg.max(axis=1, keepdims=True))
        L = e.sum(axis=1, keepdims=True)
        av = np.abs(v[bi, hi, keys])
        W = (e / L) @ av                                  # sum w |v|
        S = av.sum(axis=0)[None, :]                       # sum |v|
        eps_sum = d * L + A * len(keys)
        bo = (d * L * W + A * S + eps_sum * W) / (L - eps_sum)
        E = (eps_sum / L)[:, 0]
        bl = np.maximum(-np.log(np.maximum(1.0 - E, 1e-300)), np.log(1.0 + E))
        out[(bi, hi, i)] = (bo, bl)
    return out
