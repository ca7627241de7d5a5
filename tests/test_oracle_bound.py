"""Pins for the error scale S of the acceptance bound (CPU only).

Every GEMM parity test accepts an element when |gpu - y| <= 2^-8 |y| +
2^-12 S.  S is the scaled sum of |products| the fp32 accumulation can err
against: |s_a s_w| sum_k |a_k w_k| for the FP8 formats (ninfer PR #167,
opening summary: the scales multiply the fp32 accumulator), and for NVFP4
|t_A t_W| sum_g S^A_g S^W_g sum_{k in g} |a_k w_k| (ninfer PR #160: E2M1
codes with one E4M3 scale per 16-element K group and a tensor scale).  For
SwiGLU it carries the gate and up error scales through silu(g) u with the
largest slope of silu within the gate's error interval, so that it bounds
the effect of any errors up to those scales, not only small ones.

These tests recompute S without the oracle's code: operands decoded by
torch's float8_e4m3fn cast and by the E2M1 closed form written out here,
exact integer (or rational) sums, distinct non-unit row, column and tensor
scales, and scipy's logistic function.  A scale dropped from S, |group sum|
taken in place of the sum of |products|, or a swapped gate / up term fails
one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])


def e4m3_decode_torch(codes: np.ndarray) -> np.ndarray:
    """E4M3FN codes -> fp64 through torch's own float8_e4m3fn type."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def e2m1_decode_closed_form(nibbles: np.ndarray) -> np.ndarray:
    """E2M1 nibble -> value: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0 or 0.5)."""
    n = np.asarray(nibbles, dtype=np.int64)
    s = np.where(n & 8, -1.0, 1.0)
    e = (n >> 1) & 3
    m = n & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return s * mag


def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    c = np.empty((q.shape[0], 2 * q.shape[1]), np.int64)
    c[:, 0::2], c[:, 1::2] = q & 0xF, q >> 4
    return c


def random_scales(rng, n, lo=-9.0, hi=3.0):
    """fp32 scales far from 1 and distinct per index (log-uniform)."""
    return np.exp2(rng.uniform(lo, hi, n)).astype(np.float32)


@pytest.mark.parametrize("M,N,K", [(5, 7, 64), (3, 11, 208), (9, 4, 512)])
def test_fp8_row_S_is_scaled_sum_of_abs_products(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    W = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    sa, sw = random_scales(rng, M), random_scales(rng, N)
    D, Da = oracle.gemm_e4m3_sums(A, W)
    a, w = e4m3_decode_torch(A), e4m3_decode_torch(W)
    S_ind = np.abs(sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]) * (np.abs(a) @ np.abs(w).T)
    for epi, res in (("store", None), ("add", np.zeros((M, N), np.uint16))):
        y, S, _ = oracle.epilogue(epi, D, Da, sa, sw, res)
        np.testing.assert_allclose(S, S_ind, rtol=1e-15, atol=0)
        # and y itself is the scaled exact sum
        np.testing.assert_allclose(y, sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :] * (a @ w.T),
                                   rtol=1e-15, atol=0)


def test_fp8_tensor_S_uses_both_matrix_scales():
    rng = np.random.default_rng(21)
    A = rng.choice(FINITE, size=(4, 96)).astype(np.uint8)
    W = rng.choice(FINITE, size=(6, 96)).astype(np.uint8)
    sa, sw = np.float32(0.0173), np.float32(3.75e-4)
    D, Da = oracle.gemm_e4m3_sums(A, W)
    _, S, _ = oracle.epilogue("store", D, Da, sa, sw)
    a, w = e4m3_decode_torch(A), e4m3_decode_torch(W)
    np.testing.assert_allclose(S, abs(float(sa) * float(sw)) * (np.abs(a) @ np.abs(w).T), rtol=1e-15, atol=0)


def silu_slope(t):
    sig = expit(t)
    return sig * (1.0 + t * (1.0 - sig))


def largest_slope(lo, hi):
    """max |silu'| on [lo, hi] by dense grids refined with scipy's bounded
    scalar minimiser around the best grid point.  One grid spans the
    interval, one its part within [-40, 40] (outside it silu' is within
    1e-15 of 0 or 1)."""
    from scipy.optimize import minimize_scalar
    t = np.linspace(lo, hi, 4001)
    if max(lo, -40.0) < min(hi, 40.0):
        t = np.union1d(t, np.linspace(max(lo, -40.0), min(hi, 40.0), 4001))
    v = np.abs(silu_slope(t))
    k = int(np.argmax(v))
    a, b = t[max(k - 1, 0)], t[min(k + 1, len(t) - 1)]
    best = float(v[k])
    if b > a:
        r = minimize_scalar(lambda x: -abs(silu_slope(x)), bounds=(a, b), method="bounded",
                            options={"xatol": 1e-13 * max(1.0, abs(a))})
        best = max(best, -float(r.fun))
    return best


def test_swiglu_S_uses_the_largest_slope_in_the_gate_interval_at_non_unit_scales():
    rng = np.random.default_rng(22)
    M, Nh, K = 6, 5, 128
    A = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    W = rng.choice(FINITE, size=(2 * Nh, K)).astype(np.uint8)
    sa, sw = random_scales(rng, M, -12, -4), random_scales(rng, 2 * Nh, -12, -4)
    D, Da = oracle.gemm_e4m3_sums(A, W)
    y, S, _ = oracle.epilogue("swiglu", D, Da, sa, sw)
    a, w = e4m3_decode_torch(A), e4m3_decode_torch(W)
    s2 = sa.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    v = s2 * (a @ w.T)
    Sv = np.abs(s2) * (np.abs(a) @ np.abs(w).T)
    g, u, Sg, Su = v[:, :Nh], v[:, Nh:], Sv[:, :Nh], Sv[:, Nh:]
    silu = g * expit(g)
    np.testing.assert_allclose(y, silu * u, rtol=1e-13, atol=0)
    L = np.vectorize(lambda x, d: largest_slope(x - d, x + d))(g, 2.0 ** -12 * Sg)
    np.testing.assert_allclose(S, L * Sg * (np.abs(u) + 2.0 ** -12 * Su) + np.abs(silu) * Su, rtol=1e-9, atol=0)


@pytest.mark.parametrize("g,dg", [(2.0, 1.0), (-2.0, 1.0), (0.0, 5.0), (-13.6, 1373.0), (-767.0, 3.1e5),
                                  (7.0, 0.5), (-7.0, 0.5), (0.3, 1e-3)])
def test_swiglu_S_slope_at_interval_ends_and_inner_extrema(g, dg):
    # one element, unit scales, up = 1 exactly (Su = 0): S = L Sg, where L is
    # the largest |silu'| within 2^-12 Sg of the gate; the intervals here hold
    # the maximum of silu' (near 2.4), its minimum (near -2.4), both, or
    # neither, and the cancelling gate sums of a wide-range sweep
    Sg = dg * 4096.0
    D = np.array([[g, 1.0]])
    Da = np.array([[Sg, 0.0]])
    y, S, _ = oracle.epilogue("swiglu", D, Da, 1.0, 1.0)
    assert S[0, 0] == pytest.approx(largest_slope(g - dg, g + dg) * Sg, rel=1e-9)


def test_swiglu_S_bounds_errors_over_the_whole_interval():
    # the meaning of S: gate and up off by up to 2^-12 of their error scales,
    # anywhere in those intervals, move silu(g) u by at most 2^-12 S; the
    # gates include sums that cancel to far below their error scale
    rng = np.random.default_rng(23)
    n = 3000
    g = np.concatenate([rng.normal(0.0, 3.0, n), rng.normal(0.0, 30.0, n)])
    u = rng.normal(0.0, 2.0, 2 * n) * 10.0 ** rng.uniform(-3, 3, 2 * n)
    Sg = np.concatenate([np.abs(rng.normal(0.0, 5.0, n)) + 0.1, 10.0 ** rng.uniform(2, 7, n)])
    Su = np.abs(u) * 10.0 ** rng.uniform(0, 4, 2 * n)
    D = np.concatenate([g, u])[None, :]
    Dabs = np.concatenate([Sg, Su])[None, :]
    y, S, _ = oracle.epilogue("swiglu", D, Dabs, 1.0, 1.0)
    eps = 2.0 ** -12
    worst = 0.0
    for t in np.linspace(-1.0, 1.0, 41):
        for sgn_u in (-1.0, 1.0):
            gp, up = g + t * eps * Sg, u + sgn_u * eps * Su
            yp = gp * expit(gp) * up
            worst = max(worst, float(np.max(np.abs(yp - y[0]) / (eps * S[0]))))
    assert worst <= 1.0 + 1e-12
    assert worst >= 0.5          # and it is not loose: some element comes close


def test_nvfp4_S_is_tensor_and_block_scaled_sum_of_abs_products():
    rng = np.random.default_rng(24)
    M, N, K = 4, 5, 96
    Aq = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    Wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    pos = FINITE[(FINITE > 0) & (FINITE < 0x7F)]
    As = rng.choice(pos, size=(M, K // 16)).astype(np.uint8)
    Ws = rng.choice(pos, size=(N, K // 16)).astype(np.uint8)
    ta, tw = np.float32(1.37e-3), np.float32(2.9e-5)
    D, Da = oracle.gemm_nvfp4_sums(Aq, As, Wq, Ws)
    y, S, _ = oracle.epilogue("store", D, Da, ta, tw)
    # exact rationals: E2M1 values are multiples of 1/2, E4M3 of 2^-9
    a = e2m1_decode_closed_form(unpack_nibbles(Aq))
    w = e2m1_decode_closed_form(unpack_nibbles(Wq))
    sA, sW = e4m3_decode_torch(As), e4m3_decode_torch(Ws)
    mixed_groups = 0
    for i in range(M):
        for j in range(N):
            tot, tot_abs = Fraction(0), Fraction(0)
            for gi in range(K // 16):
                ks = slice(16 * gi, 16 * gi + 16)
                p = [Fraction(x) * Fraction(z) for x, z in zip(a[i, ks], w[j, ks])]
                sc = Fraction(sA[i, gi]) * Fraction(sW[j, gi])
                tot += sc * sum(p)
                tot_abs += sc * sum(abs(x) for x in p)
                mixed_groups += int(any(x > 0 for x in p) and any(x < 0 for x in p))
            t2 = Fraction(float(ta)) * Fraction(float(tw))
            assert abs(Fraction(S[i, j]) - t2 * tot_abs) <= Fraction(2) ** -48 * t2 * tot_abs
            assert abs(Fraction(y[i, j]) - t2 * tot) <= Fraction(2) ** -48 * t2 * tot_abs
    assert mixed_groups > 0      # |group sum| < sum of |products| somewhere


def test_bound_rejects_errors_twice_its_size_on_a_real_output():
    # errors of 2^-7 |y| + 2^-11 S placed on top of the oracle's own rounded
    # output, away from y, leave the bound everywhere y or S is nonzero
    rng = np.random.default_rng(25)
    A = rng.choice(FINITE, size=(8, 256)).astype(np.uint8)
    W = rng.choice(FINITE, size=(12, 256)).astype(np.uint8)
    sa, sw = random_scales(rng, 8), random_scales(rng, 12)
    D, Da = oracle.gemm_e4m3_sums(A, W)
    y, S, out = oracle.epilogue("store", D, Da, sa, sw)
    g = oracle.bf16_to_f64(out)
    away = np.where(g >= y, 1.0, -1.0)
    bad_vals = g + away * (2.0 ** -7 * np.abs(y) + 2.0 ** -11 * S)
    bad = np.vectorize(oracle.bf16_from_f64, otypes=[np.uint16])(bad_vals)
    ok, _ = oracle.within_tolerance(bad, y, S)
    assert not ok.any()
