"""Pins for the oracle's quantizers (CPU only).

What fixes the expected values: the per-row scale amax/448 (row-scaled FP8 of
ninfer PR #167), the per-matrix scale (AstrAI's per-tensor NT benchmark), the
NVFP4 layout (E2M1 codes, E4M3 scale per 16 K-elements, fp32 tensor scale,
ninfer PR #160) and the readings stated in the oracle's header.  Each test
compares against a separately written brute force (numpy float32 steps plus
exhaustive nearest-value search), a library cast, or an invariant the
definition forces.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_normal, f32_to_bf16_bits

E4 = oracle.E4M3_TABLE
E2 = oracle.E2M1_TABLE


def _nearest(vals, mags):
    a = np.minimum(np.abs(vals.astype(np.float64)), 2 * mags.max())[:, None]
    d = np.abs(a - mags[None, :])
    best = []
    for row in d:
        m = row.min()
        c = np.nonzero(row == m)[0]
        even = [i for i in c if i % 2 == 0]
        best.append(even[0] if even else c[0])
    return np.array(best)


def brute_rowwise(x16):
    """numpy float32 steps + exhaustive search; independent of oracle.c."""
    x = (x16.astype(np.uint32) << 16).view(np.float32)
    q = np.zeros(x.shape, np.int64)
    s = np.zeros(x.shape[0], np.float32)
    for r in range(x.shape[0]):
        amax = np.float32(np.max(np.abs(x[r]))) if x.shape[1] else np.float32(0)
        s[r] = amax / np.float32(448.0)
        if s[r] > 0:
            ratio = x[r] / s[r]
            q[r] = _nearest(ratio, E4[:127]) | np.where(np.signbit(ratio), 0x80, 0)
        else:
            q[r] = np.where(np.signbit(x[r]), 0x80, 0)
    return q, s


@pytest.mark.parametrize("shape", [(1, 16), (3, 32), (5, 48), (7, 64)])
def test_rowwise_vs_brute_force(shape):
    x = bf16_normal(shape, 1.0, 11 + shape[0])
    q, s = oracle.quantize_rowwise(x)
    qb, sb = brute_rowwise(x)
    assert np.array_equal(s.view(np.uint32), sb.view(np.uint32))
    assert np.array_equal(q.astype(np.int64), qb)


def test_rowwise_amax_element_encodes_to_448():
    x = bf16_normal((64, 512), 1.0, 3)
    q, s = oracle.quantize_rowwise(x)
    xf = oracle.bf16_to_f64(x)
    idx = np.argmax(np.abs(xf), axis=1)
    top = q[np.arange(64), idx]
    assert np.all((top == 0x7E) | (top == 0xFE))
    assert np.all((top == 0xFE) == (xf[np.arange(64), idx] < 0))


def test_rowwise_power_of_two_scale_is_exact():
    # rows of exact E4M3 values times 2^k with 448 * 2^k present: s = 2^k and
    # every code reproduces its value exactly
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    for k in (-20, -3, 0, 4, 11):
        codes = rng.choice(finite, size=(4, 64))
        codes[:, 7] = 0x7E
        vals = E4[codes] * 2.0 ** k
        x16 = f32_to_bf16_bits(vals.astype(np.float32))
        assert np.array_equal(oracle.bf16_to_f64(x16), vals)     # exact in bf16
        q, s = oracle.quantize_rowwise(x16)
        assert np.all(s == np.float32(2.0 ** k))
        assert np.array_equal(E4[q] * 2.0 ** k, vals)


def test_rowwise_zero_row_and_signed_zeros():
    x = np.zeros((2, 32), np.uint16)
    x[1, ::2] = 0x8000          # -0.0
    q, s = oracle.quantize_rowwise(x)
    assert np.all(s == 0)
    assert np.all(q[0] == 0)
    assert np.all(q[1, ::2] == 0x80) and np.all(q[1, 1::2] == 0)


def test_rowwise_matches_torch_cast_of_the_ratio():
    x = bf16_normal((32, 256), 1.0, 8)
    q, s = oracle.quantize_rowwise(x)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    ratio = xf / s[:, None]                      # float32 IEEE division
    ref = torch.from_numpy(np.ascontiguousarray(ratio)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_rowwise_dequant_error_is_half_an_e4m3_step():
    x = bf16_normal((16, 512), 1.0, 9)
    q, s = oracle.quantize_rowwise(x)
    xf = oracle.bf16_to_f64(x)
    deq = E4[q] * s[:, None].astype(np.float64)
    r = np.abs(xf) / s[:, None]
    # step of E4M3 around r: 2^(floor(log2 r) - 3), at least 2^-9 (subnormals)
    step = np.where(r >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(r, 1e-300))) - 3), 2.0 ** -9)
    # fl32(x/s) adds at most one fp32 rounding on top of the E4M3 half step
    bound = (0.5 * step + r * 2.0 ** -24) * s[:, None]
    assert np.all(np.abs(deq - xf) <= bound * (1 + 1e-12))


def test_tensor_quant_batch_vs_brute_force():
    x = bf16_normal((3, 5, 32), 1.0, 21)
    q, s = oracle.quantize_tensor(x)
    for b in range(3):
        xf = (x[b].astype(np.uint32) << 16).view(np.float32)
        sb = np.float32(np.max(np.abs(xf))) / np.float32(448.0)
        assert s[b].view(np.uint32) == sb.view(np.uint32)
        ratio = (xf / sb).ravel()
        ref = _nearest(ratio, E4[:127]) | np.where(np.signbit(ratio), 0x80, 0)
        assert np.array_equal(q[b].ravel().astype(np.int64), ref)


def test_rows_with_scale_reproduces_tensor_quant():
    x = bf16_normal((40, 64), 1.0, 22)
    q, s = oracle.quantize_tensor(x)
    q2 = oracle.quantize_rows_with_scale(x[10:17], s[0])
    assert np.array_equal(q2, q[10:17])


# --------------------------------------------------------------------------
# NVFP4
# --------------------------------------------------------------------------

def brute_block16(x16):
    x = (x16.astype(np.uint32) << 16).view(np.float32)
    R, K = x.shape
    t = np.float32(np.max(np.abs(x))) / np.float32(2688.0)
    six_t = np.float32(6.0) * t
    codes = np.zeros((R, K), np.int64)
    bsc = np.zeros((R, K // 16), np.int64)
    for r in range(R):
        for g in range(K // 16):
            blk = x[r, 16 * g:16 * g + 16]
            amax_g = np.float32(np.max(np.abs(blk)))
            b = int(_nearest(np.array([amax_g / six_t], np.float32), E4[:127])[0]) if t > 0 else 0
            bsc[r, g] = b
            e = np.float32(E4[b]) * t
            if e > 0:
                ratio = blk / e
                codes[r, 16 * g:16 * g + 16] = _nearest(ratio, E2[:8]) | np.where(np.signbit(ratio), 8, 0)
            else:
                codes[r, 16 * g:16 * g + 16] = np.where(np.signbit(blk), 8, 0)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, bsc.astype(np.uint8), t


@pytest.mark.parametrize("shape,std", [((2, 32), 1.0), ((3, 64), 0.02), ((4, 96), 3.0)])
def test_block16_vs_brute_force(shape, std):
    x = bf16_normal(shape, std, 31 + shape[0])
    q, bs, t = oracle.quantize_block16(x)
    qb, bsb, tb = brute_block16(x)
    assert np.float32(t).view(np.uint32) == np.float32(tb).view(np.uint32)
    assert np.array_equal(bs, bsb)
    assert np.array_equal(q, qb)


def test_block16_tensor_amax_block_scale_is_448_and_elements_reach_6():
    x = bf16_normal((32, 256), 1.0, 41)
    q, bs, t = oracle.quantize_block16(x)
    xf = oracle.bf16_to_f64(x)
    r, c = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    assert bs[r, c // 16] == 0x7E
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(xf.shape)
    # block maxima encode to +-6 whenever the block scale is a normal E4M3
    for rr in range(32):
        for g in range(16):
            if bs[rr, g] >= 0x08:
                blk = np.abs(xf[rr, 16 * g:16 * g + 16])
                k = 16 * g + int(np.argmax(blk))
                assert codes[rr, k] & 0x7 == 7


def test_block16_nibble_order_and_dequant_bound():
    x = bf16_normal((8, 64), 1.0, 43)
    q, bs, t = oracle.quantize_block16(x)
    xf = oracle.bf16_to_f64(x)
    lo, hi = E2[q & 0xF], E2[q >> 4]
    vals = np.empty(xf.shape)
    vals[:, 0::2], vals[:, 1::2] = lo, hi
    S = np.repeat(E4[bs], 16, axis=1)
    deq = vals * S * float(t)
    # within half an E2M1 step (<= 1 at the top of the range) of x / (S t), relative
    # to the per-block scale, plus fp32 roundings of S*t and x/(S*t)
    e = S * float(t)
    assert np.all(np.abs(deq - xf) <= e * 1.0 + np.abs(xf) * 2.0 ** -20 + 1e-30)
    # sign of zero kept: a zero input's nibble carries its sign
    x2 = x.copy()
    x2[0, 0] = 0x8000
    q2, _, _ = oracle.quantize_block16(x2)
    assert q2[0, 0] & 0xF == 0x8


def test_block16_zero_tensor():
    x = np.zeros((4, 32), np.uint16)
    x[1, 3] = 0x8000
    q, bs, t = oracle.quantize_block16(x)
    assert t == 0 and np.all(bs == 0)
    assert (q[1, 1] >> 4) == 0x8 and np.count_nonzero(q) == 1


def test_block16_rows_reproduce_whole_tensor():
    x = bf16_normal((20, 64), 1.0, 44)
    q, bs, t = oracle.quantize_block16(x)
    q2, bs2 = oracle.quantize_block16_rows(x[5:9], t)
    assert np.array_equal(q2, q[5:9]) and np.array_equal(bs2, bs[5:9])
