"""Pins of the oracle's FP8 (e4m3) pieces: the rounding against PyTorch's float8_e4m3fn
conversion, the code table, the quantization layouts, and the probability-cast error bound
against a brute-force simulation of the cast."""
import numpy as np
import pytest
import torch

from oracle import fp8
from oracle.bsa_oracle import num_blocks


def test_rounding_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(50000).astype(np.float32) * s
                        for s in (1e-4, 1e-2, 1, 30, 120)])
    x = x[np.abs(x) <= 448]
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    bf = (bits << 16).view(np.float32)
    bf = bf[np.isfinite(bf) & (np.abs(bf) <= 448)]              # every bf16 value in range
    vals = fp8.e4m3_decode(np.arange(0, 127, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # every tie
    allx = np.concatenate([x, bf, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(allx).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_round(allx), ref)


def test_code_table():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    v = fp8.e4m3_decode(codes)
    assert np.array_equal(fp8.e4m3_round(v.astype(np.float32))[v != 0], codes[v != 0])
    assert fp8.e4m3_decode(np.uint8(0x7E)) == 448.0
    assert fp8.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9       # smallest subnormal
    assert fp8.e4m3_decode(np.uint8(0x08)) == 2.0 ** -6       # smallest normal
    assert fp8.e4m3_decode(np.uint8(0x38)) == 1.0
    with pytest.raises(ValueError):
        fp8.e4m3_round(np.float32(465.0))


def _bf16_bits(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_quantize_rows_scale_and_error():
    rng = np.random.default_rng(1)
    B, D = 64, 64
    x = rng.standard_normal((2, 3, 3 * B, D)) * np.array([0.01, 1.0, 50.0])[None, :, None, None]
    x[1, 2, B:2 * B] = 0.0                                       # an all-zero block
    bits = _bf16_bits(x)
    xv = fp8.widen_bf16(bits)
    codes, s = fp8.quantize_rows(bits, B)
    assert s[1, 2, 1] == 0 and not codes[1, 2, B:2 * B].any()
    deq = fp8.dequantize_rows(codes, s, B)
    for bi in range(2):
        for hi in range(3):
            for j in range(3):
                blk = xv[bi, hi, j * B:(j + 1) * B]
                amax = np.abs(blk).max()
                if amax == 0:
                    continue
                # the largest entry lands on the top code 448
                assert np.abs(fp8.e4m3_decode(codes[bi, hi, j * B:(j + 1) * B])).max() == 448.0
                assert s[bi, hi, j] == np.float32(np.float32(amax) / np.float32(448))
                err = np.abs(deq[bi, hi, j * B:(j + 1) * B] - blk)
                # half an ulp: 2^-4 relative (normal codes) or 2^-10 codes (subnormal)
                assert np.all(err <= 2.0 ** -4 * np.abs(blk) * 1.0001 + 2.0 ** -10 * s[bi, hi, j])


def test_quantize_v_one_scale_per_head():
    """V takes one scale per (batch, head): the same codes and scale as quantizing the whole
    head as one block; dequantized within half an E4M3 ulp; a head of zeros gets scale 0."""
    rng = np.random.default_rng(2)
    B, D = 128, 64
    x = rng.standard_normal((2, 3, 2 * B, D)) * np.array([0.02, 1.0, 40.0])[None, :, None, None]
    x[1, 0] = 0.0
    bits = _bf16_bits(x)
    codes, s = fp8.quantize_v(bits, B)
    assert codes.shape == (2, 3, 2 * B, D) and s.shape == (2, 3)
    c_one, s_one = fp8.quantize_rows(bits, 2 * B)                # one block = the whole head
    assert np.array_equal(codes, c_one) and np.array_equal(s, s_one[:, :, 0])
    assert s[1, 0] == 0 and not codes[1, 0].any()
    xv = fp8.widen_bf16(bits)
    for bi in range(2):
        for hi in range(3):
            if s[bi, hi] == 0:
                continue
            assert np.abs(fp8.e4m3_decode(codes[bi, hi])).max() == 448.0
    deq = fp8.dequantize_v(codes, s)
    assert np.all(np.abs(deq - xv) <= 2.0 ** -4 * np.abs(xv) * 1.0001
                  + 2.0 ** -10 * s[:, :, None, None])


def test_v8_layout_helper_is_a_bijection():
    """The test-side map between the library's block-transposed V codes and the token-major
    codes of the oracle: inverse of each other, and the first positions of a row hold the keys
    the header lists for them."""
    from fp8_support import tokens_to_v8, v8_key_order, v8_to_tokens
    B, D = 128, 128
    order = v8_key_order(B)
    assert sorted(order.tolist()) == list(range(B))
    # bytes 0..15 of half 0: keys 0-3, 8-11, 16-19, 24-27; bytes 32..47 (half 1): +4
    assert order[:16].tolist() == [8 * g + u for g in range(4) for u in range(4)]
    assert order[32:48].tolist() == [8 * g + 4 + u for g in range(4) for u in range(4)]
    assert order[64:80].tolist() == [64 + 8 * g + u for g in range(4) for u in range(4)]
    rng = np.random.default_rng(5)
    tok = rng.integers(0, 255, size=(1, 2, 3 * B, D), dtype=np.uint8)
    v8 = tokens_to_v8(tok, B)
    assert v8.shape == (1, 2, 3, D, B)
    assert v8[0, 1, 2, 5, 7] == tok[0, 1, 2 * B + order[7], 5]
    assert np.array_equal(v8_to_tokens(v8), tok)


def test_error_bound_holds_for_simulated_cast():
    """Brute force: run the online softmax block by block in the column order with the
    probabilities cast to E4M3 as 2^8 exp(l - m_running), and check the result against the
    exact attention within attn_error_bound."""
    rng = np.random.default_rng(3)
    B, D, N = 64, 64, 5 * 64 - 7
    n = num_blocks(N, B)
    Np = n * B
    q = rng.standard_normal((1, 1, Np, D)) * 1.5
    k = rng.standard_normal((1, 1, Np, D))
    v = rng.standard_normal((1, 1, Np, D)) * 3
    for t in (q, k, v):
        t[:, :, N:] = 0
    scale = 1 / np.sqrt(D)
    row_ptr = np.array([0, 5, 7, 10, 11, 16])
    col_idx = np.array([0, 1, 2, 3, 4, 1, 3, 0, 2, 4, 2, 0, 1, 2, 3, 4])
    rows = [(0, 0, i) for i in range(n)]
    bound = fp8.attn_error_bound(q, k, v, row_ptr, col_idx, N, B, scale, rows)
    worst = 0.0
    for (_, _, i) in rows:
        lo, hi = i * B, min((i + 1) * B, N)
        acc = np.zeros((hi - lo, D))
        lsum = np.zeros((hi - lo, 1))
        m = np.full((hi - lo, 1), -np.inf)
        keys_all = []
        for j in col_idx[row_ptr[i]:row_ptr[i + 1]]:
            keys = np.arange(j * B, min((j + 1) * B, N))
            keys_all.append(keys)
            lg = scale * (q[0, 0, lo:hi] @ k[0, 0, keys].T)
            mn = np.maximum(m, lg.max(axis=1, keepdims=True))
            a = np.exp(m - mn)
            e = 2.0 ** 8 * np.exp(lg - mn)
            p8 = fp8.e4m3_decode(fp8.e4m3_round(e.astype(np.float32)))
            acc = acc * a + p8 @ v[0, 0, keys]
            lsum = lsum * a + e.sum(axis=1, keepdims=True)
            m = mn
        keys = np.concatenate(keys_all)
        lg = scale * (q[0, 0, lo:hi] @ k[0, 0, keys].T)
        w = np.exp(lg - lg.max(axis=1, keepdims=True))
        exact = (w / w.sum(axis=1, keepdims=True)) @ v[0, 0, keys]
        err = np.abs(acc / lsum - exact)
        assert np.all(err <= bound[(0, 0, i)])
        worst = max(worst, float((err / bound[(0, 0, i)]).max()))
    assert worst > 0.01            # the bound is not vacuous by orders of magnitude


@pytest.mark.parametrize("rounding", ["nearest", "floor"])
def test_expcast_codes_and_bound(rounding):
    """ExpCast codes: exact powers of two map to their E4M3 codes; and a brute-force online
    softmax with the probabilities cast by ExpCast (either rounding of the byte conversion)
    stays within expcast_error_bound, output and lse."""
    y = np.arange(-6, 9, dtype=np.float64)                    # 2^y, normal range
    ref = torch.from_numpy((2.0 ** y).astype(np.float32)).to(torch.float8_e4m3fn)
    assert np.array_equal(fp8.expcast_codes(y, rounding), ref.view(torch.uint8).numpy())
    assert fp8.expcast_codes(np.array([-np.inf]), rounding)[0] == 0
    rng = np.random.default_rng(4)
    B, D, N = 64, 64, 6 * 64 - 5
    n = num_blocks(N, B)
    Np = n * B
    q = rng.standard_normal((1, 1, Np, D)) * 2.0
    k = rng.standard_normal((1, 1, Np, D))
    v = rng.standard_normal((1, 1, Np, D)) * 3
    for t in (q, k, v):
        t[:, :, N:] = 0
    scale = 1 / np.sqrt(D)
    row_ptr = np.array([0, 6, 8, 11, 12, 16, 19])
    col_idx = np.array([0, 1, 2, 3, 4, 5, 1, 3, 0, 2, 4, 2, 0, 1, 2, 3, 5, 4, 3])
    rows = [(0, 0, i) for i in range(n)]
    bound = fp8.expcast_error_bound(q, k, v, row_ptr, col_idx, N, B, scale, rows)
    worst = 0.0
    for (_, _, i) in rows:
        lo, hi = i * B, min((i + 1) * B, N)
        acc = np.zeros((hi - lo, D))
        lsum = np.zeros((hi - lo, 1))
        m = np.full((hi - lo, 1), -np.inf)
        keys_all = []
        for j in col_idx[row_ptr[i]:row_ptr[i + 1]]:
            keys = np.arange(j * B, min((j + 1) * B, N))
            keys_all.append(keys)
            lg = scale * (q[0, 0, lo:hi] @ k[0, 0, keys].T)
            mn = np.maximum(m, lg.max(axis=1, keepdims=True))
            a = np.exp(m - mn)
            y = (lg - mn) / np.log(2) + 8                      # log2 of 2^8 exp(l - m)
            p8 = fp8.e4m3_decode(fp8.expcast_codes(y, rounding))
            acc = acc * a + p8 @ v[0, 0, keys]
            lsum = lsum * a + p8.sum(axis=1, keepdims=True)
            m = mn
        keys = np.concatenate(keys_all)
        lg = scale * (q[0, 0, lo:hi] @ k[0, 0, keys].T)
        mx = lg.max(axis=1, keepdims=True)
        w = np.exp(lg - mx)
        exact = (w / w.sum(axis=1, keepdims=True)) @ v[0, 0, keys]
        lse = (mx + np.log(w.sum(axis=1, keepdims=True)))[:, 0]
        lse_cast = (m[:, 0] + np.log(lsum[:, 0] / 2.0 ** 8))
        bo, bl = bound[(0, 0, i)]
        err = np.abs(acc / lsum - exact)
        assert np.all(err <= bo)
        assert np.all(np.abs(lse_cast - lse) <= bl)
        worst = max(worst, float((err / bo).max()))
    assert worst > 0.01
