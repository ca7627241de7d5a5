"""Pins for the oracle's GEMM, scale application, epilogues and acceptance
bound (CPU only).

The method (ninfer PR #167 opening summary): fp32 accumulation of FP8 code
products, then the scales, then one of the linear / linear_add /
linear_swiglu epilogues, bf16 out.  Pins: exact integer arithmetic on the
codes' integer mantissas, naive triple loops, numpy matmul of dequantized
operands, scipy's logistic function for SiLU, and special cases (zero,
identity and one-hot weights) whose outputs are known in closed form.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
from synthetic import bf16_normal, f32_to_bf16_bits

E4 = oracle.E4M3_TABLE
E2 = oracle.E2M1_TABLE
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])


def test_e4m3_sums_equal_exact_integer_dot_products():
    rng = np.random.default_rng(1)
    A = rng.choice(FINITE, size=(9, 640)).astype(np.uint8)
    W = rng.choice(FINITE, size=(13, 640)).astype(np.uint8)
    D, Da = oracle.gemm_e4m3_sums(A, W)
    ai = (E4[A] * 512).astype(np.int64)      # integer multiples of 2^-9
    wi = (E4[W] * 512).astype(np.int64)
    assert np.array_equal(ai, E4[A] * 512) and np.array_equal(wi, E4[W] * 512)
    exact = ai @ wi.T                          # int64, no overflow at these K
    assert np.array_equal(D * 2.0 ** 18, exact.astype(np.float64))
    assert np.array_equal(Da * 2.0 ** 18, (np.abs(ai) @ np.abs(wi).T).astype(np.float64))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 2, 17), (4, 6, 33)])
def test_e4m3_sums_vs_naive_loop(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    A = rng.choice(FINITE, size=(M, K)).astype(np.uint8)
    W = rng.choice(FINITE, size=(N, K)).astype(np.uint8)
    D, Da = oracle.gemm_e4m3_sums(A, W)
    for i in range(M):
        for j in range(N):
            s = sum(E4[A[i, k]] * E4[W[j, k]] for k in range(K))
            assert D[i, j] == s


def test_full_path_vs_naive_loop_with_distinct_row_scales():
    # a transposed operand, a swapped scale index or a dropped scale fails here
    A16 = bf16_normal((5, 48), 1.0, 2)
    W16 = bf16_normal((7, 48), 0.02, 3)
    A16[1] = f32_to_bf16_bits(oracle.bf16_to_f64(A16[1]).astype(np.float32) * 64)
    res = oracle.linear_e4m3_rowwise(A16, W16, "store")
    Aq, sa, Wq, sw = res["Aq"], res["sa"], res["Wq"], res["sw"]
    for i in range(5):
        for j in range(7):
            ref = float(sa[i]) * float(sw[j]) * sum(E4[Aq[i, k]] * E4[Wq[j, k]] for k in range(48))
            assert res["y"][i, j] == pytest.approx(ref, rel=1e-15, abs=0)
            assert res["out"][i, j] == oracle.bf16_from_f64(ref)


def test_gemm_close_to_unquantized_product():
    # quantization error only: the row-scaled E4M3 product tracks the bf16 product
    A16 = bf16_normal((16, 256), 1.0, 4)
    W16 = bf16_normal((24, 256), 0.02, 5)
    res = oracle.linear_e4m3_rowwise(A16, W16, "store")
    exact = oracle.bf16_to_f64(A16) @ oracle.bf16_to_f64(W16).T
    assert np.max(np.abs(res["y"] - exact)) < 0.05 * np.max(np.abs(exact))


def test_identity_weight_returns_dequantized_activations():
    K = 64
    A16 = bf16_normal((6, K), 1.0, 6)
    W16 = f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    res = oracle.linear_e4m3_rowwise(A16, W16, "store")
    # each identity row quantizes to a single 448 code with scale fl32(1/448)
    deq = E4[res["Aq"]] * res["sa"][:, None].astype(np.float64)
    sw = res["sw"].astype(np.float64)
    assert np.all(res["Wq"][np.arange(K), np.arange(K)] == 0x7E)
    assert np.allclose(res["y"], deq * 448.0 * sw[None, :], rtol=0, atol=0)


def test_one_hot_weight_selects_columns():
    rng = np.random.default_rng(7)
    M, N, K = 9, 11, 80
    A16 = bf16_normal((M, K), 1.0, 8)
    pick = rng.integers(0, K, N)
    Wf = np.zeros((N, K), np.float32)
    Wf[np.arange(N), pick] = 2.0
    res = oracle.linear_e4m3_rowwise(A16, f32_to_bf16_bits(Wf), "store")
    deqA = E4[res["Aq"]] * res["sa"][:, None].astype(np.float64)
    expect = deqA[:, pick] * (448.0 * res["sw"].astype(np.float64))[None, :]
    assert np.array_equal(res["y"], expect)


def test_zero_weight_add_returns_residual_bitwise():
    A16 = bf16_normal((8, 32), 1.0, 9)
    W16 = np.zeros((12, 32), np.uint16)
    R16 = bf16_normal((8, 12), 1.0, 10)
    res = oracle.linear_e4m3_rowwise(A16, W16, "add", residual=R16)
    assert np.array_equal(res["out"], R16)
    assert np.all(res["S"] == 0)


def test_bias_row_adds_to_every_token_row():
    # the bf16 bias epilogue is the residual add with one row broadcast to
    # every token row (AstrAI commit log for gemm.cuh, the commit fusing the
    # bias): zero weights give the bias itself in every row, bit for bit, and
    # otherwise y is the store result plus the bias value of the column
    A16 = bf16_normal((8, 32), 1.0, 13)
    bias = bf16_normal((12,), 1.0, 14)
    R = np.broadcast_to(bias, (8, 12))
    z = oracle.linear_e4m3_rowwise(A16, np.zeros((12, 32), np.uint16), "add", residual=R)
    assert np.array_equal(z["out"], np.tile(bias, (8, 1)))
    W16 = bf16_normal((12, 32), 0.02, 15)
    b = oracle.linear_e4m3_rowwise(A16, W16, "add", residual=R)
    st = oracle.linear_e4m3_rowwise(A16, W16, "store")
    bias_f = (bias.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(b["y"], st["y"] + bias_f[None, :])


def _bf16_val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_e4m3_bias_values_by_hand():
    # E4M3 bias codes times one fp32 scale (AstrAI commit log, the commit
    # fusing the bias: FP8 bias storage dequantized in the epilogue).  Code
    # values worked by hand: sign, 4 exponent bits (bias 7), 3 mantissa bits.
    codes = np.array([0x38, 0xB8, 0x3C, 0x44, 0x7E, 0xFE, 0x08, 0x01, 0x00, 0x80], np.uint8)
    want = np.array([1.0, -1.0, 1.5, 3.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 0.0, -0.0])
    assert np.array_equal(oracle.bias_e4m3(codes, 1.0), want)
    assert np.array_equal(oracle.bias_e4m3(codes, 0.75), want * 0.75)
    # the scale is taken as fp32: 0.1 becomes float32(0.1), not the double
    assert oracle.bias_e4m3(np.array([0x38], np.uint8), 0.1)[0] == float(np.float32(0.1))


def test_e4m3_bias_with_zero_weights_is_its_nearest_bf16():
    # zero weights: every row of the output is bf16(dec(code) * scale), one
    # rounding of the exact product (checked against both bf16 neighbours)
    A16 = bf16_normal((6, 32), 1.0, 21)
    rng = np.random.default_rng(22)
    codes = rng.choice(FINITE, size=(12,)).astype(np.uint8)
    scale = np.float32(1.0 / 3.0)
    exact = E4[codes] * np.float64(scale)
    z = oracle.linear_e4m3_rowwise(A16, np.zeros((12, 32), np.uint16), "add",
                                   bias=oracle.bias_e4m3(codes, scale))
    assert np.array_equal(z["out"], np.tile(z["out"][0], (6, 1)))
    got = z["out"][0]
    err = np.abs(_bf16_val(got) - exact)
    for nb in (got.astype(np.int64) + 1, got.astype(np.int64) - 1):
        nb_val = _bf16_val((nb & 0xFFFF).astype(np.uint16))
        assert np.all(err <= np.abs(nb_val - exact))
    assert np.array_equal(np.signbit(_bf16_val(got)) | (exact == 0), np.signbit(exact) | (exact == 0))


def test_e4m3_bias_adds_after_the_operand_scales():
    # with weights: y is the store result plus the dequantized bias of the
    # column (not scaled by sa sw, not indexed by row), in fp64 exactly; a
    # bias made by row-quantizing a bf16 row is that row within E4M3's
    # half-ulp (2^-4 relative, or 2^-10 of the row's scale for subnormals)
    A16 = bf16_normal((8, 64), 1.0, 23)
    W16 = bf16_normal((12, 64), 0.02, 24)
    row = bf16_normal((12,), 0.5, 25)
    bq, bs = oracle.quantize_rowwise(row[None, :])
    b = oracle.bias_e4m3(bq[0], bs[0])
    rv = _bf16_val(row)
    assert np.all(np.abs(b - rv) <= 2.0 ** -4 * np.abs(rv) + 2.0 ** -10 * float(bs[0]))
    res = oracle.linear_e4m3_rowwise(A16, W16, "add", bias=b)
    st = oracle.linear_e4m3_rowwise(A16, W16, "store")
    assert np.array_equal(res["y"], st["y"] + b[None, :])
    assert np.array_equal(res["S"], st["S"])
    # a bias of exact bf16 values (scale 1) equals the bf16 bias row
    c1 = np.array([0x38, 0xC0, 0x30, 0x01, 0x7E, 0x00, 0xB4, 0x4A, 0x3A, 0x22, 0x9F, 0x5C], np.uint8)
    row1 = f32_to_bf16_bits(E4[c1].astype(np.float32))
    r1 = oracle.linear_e4m3_rowwise(A16, W16, "add", residual=np.broadcast_to(row1, (8, 12)))
    b1 = oracle.linear_e4m3_rowwise(A16, W16, "add", bias=oracle.bias_e4m3(c1, 1.0))
    assert np.array_equal(r1["out"], b1["out"]) and np.array_equal(r1["y"], b1["y"])


def test_swiglu_matches_scipy_logistic_and_pairs_rows():
    A16 = bf16_normal((6, 64), 1.0, 11)
    W16 = bf16_normal((10, 64), 0.02, 12)
    res = oracle.linear_e4m3_rowwise(A16, W16, "swiglu")
    st = oracle.linear_e4m3_rowwise(A16, W16, "store")
    v = st["y"]
    gate, up = v[:, :5], v[:, 5:]
    expect = gate * expit(gate) * up
    assert res["y"].shape == (6, 5)
    assert np.allclose(res["y"], expect, rtol=1e-14, atol=0)


def test_swiglu_special_values():
    D = np.array([[0.0, 50.0, -50.0, 3.0, 2.0, 5.0]])   # gate | up, Nout = 3
    Da = np.array([[4.0, 50.0, 50.0, 3.0, 2.0, 8.0]])
    y, S, out = oracle.epilogue("swiglu", D, Da, 1.0, 1.0)
    assert y[0, 0] == 0.0                                   # silu(0) = 0
    assert y[0, 1] == pytest.approx(50.0 * 2.0, rel=1e-20)  # silu(z) ~ z for large z
    assert abs(y[0, 2]) < 1e-19                             # silu(-50) ~ 0
    # error scale L Sg (|u| + 2^-12 Su) + |silu(g)| Su, L the largest |silu'|
    # within 2^-12 Sg of g: silu' rises through 1/2 at 0 and falls towards 1
    # above 2.4, so L is taken at the interval's upper end, then its lower end
    dsilu = lambda z: expit(z) * (1 + z * (1 - expit(z)))
    assert S[0, 0] == pytest.approx(dsilu(4.0 / 4096) * 4.0 * (3.0 + 3.0 / 4096), rel=1e-15)
    z = 50.0
    assert S[0, 1] == pytest.approx(dsilu(z - 50.0 / 4096) * 50.0 * (2.0 + 2.0 / 4096) + z * expit(z) * 2.0,
                                    rel=1e-15)


def test_tensor_scale_epilogue_store():
    A16 = bf16_normal((2, 4, 32), 1.0, 13)
    B16 = bf16_normal((2, 6, 32), 1.0, 14)
    qa, sa = oracle.quantize_tensor(A16)
    qb, sb = oracle.quantize_tensor(B16)
    for b in range(2):
        D, Da = oracle.gemm_e4m3_sums(qa[b], qb[b])
        y, S, out = oracle.epilogue("store", D, Da, sa[b], sb[b])
        ref = (E4[qa[b]] * float(sa[b])) @ (E4[qb[b]] * float(sb[b])).T
        assert np.allclose(y, ref, rtol=1e-14, atol=0)


def test_nvfp4_sums_equal_exact_integers():
    rng = np.random.default_rng(15)
    M, N, K = 5, 7, 96
    Aq = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    Wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    As = rng.choice(FINITE[FINITE < 0x7F], size=(M, K // 16)).astype(np.uint8)   # positive scales
    Ws = rng.choice(FINITE[FINITE < 0x7F], size=(N, K // 16)).astype(np.uint8)
    D, Da = oracle.gemm_nvfp4_sums(Aq, As, Wq, Ws)

    def ints(q):
        c = np.empty((q.shape[0], 2 * q.shape[1]), np.int64)
        c[:, 0::2], c[:, 1::2] = q & 0xF, q >> 4
        return (E2[c] * 2).astype(np.int64)          # E2M1 values are multiples of 1/2

    ai, wi = ints(Aq), ints(Wq)
    sa, sw = (E4[As] * 512).astype(np.int64), (E4[Ws] * 512).astype(np.int64)
    for i in range(M):
        for j in range(N):
            exact = sum(int(sa[i, g]) * int(sw[j, g]) * int(ai[i, 16 * g:16 * g + 16] @ wi[j, 16 * g:16 * g + 16])
                        for g in range(K // 16))
            # D is exact up to fp64 rounding of the sum of scaled group terms
            assert abs(D[i, j] * 2.0 ** 20 - exact) <= 2.0 ** -50 * Da[i, j] * 2.0 ** 20 + 0


def test_nvfp4_full_path_vs_dequantized_matmul():
    A16 = bf16_normal((12, 128), 1.0, 16)
    W16 = bf16_normal((10, 128), 0.02, 17)
    qa, bsa, ta = oracle.quantize_block16(A16)
    qw, bsw, tw = oracle.quantize_block16(W16)
    D, Da = oracle.gemm_nvfp4_sums(qa, bsa, qw, bsw)
    y, S, out = oracle.epilogue("store", D, Da, ta, tw)

    def deq(q, bs, t):
        c = np.empty((q.shape[0], 2 * q.shape[1]), np.int64)
        c[:, 0::2], c[:, 1::2] = q & 0xF, q >> 4
        return E2[c] * np.repeat(E4[bs], 16, axis=1) * float(t)

    ref = deq(qa, bsa, ta) @ deq(qw, bsw, tw).T
    assert np.allclose(y, ref, rtol=1e-13, atol=1e-300)
    # and the quantized product tracks the bf16 product (NVFP4 is coarse)
    exact = oracle.bf16_to_f64(A16) @ oracle.bf16_to_f64(W16).T
    assert np.max(np.abs(y - exact)) < 0.25 * np.max(np.abs(exact))


def test_acceptance_bound_accepts_rounding_and_rejects_planted_errors():
    y = np.array([[1.0, -3.0, 100.0, 0.0]])
    S = np.array([[10.0, 10.0, 10.0, 16.0]])
    good = np.array([[oracle.bf16_from_f64(v) for v in y[0]]], np.uint16)
    ok, _ = oracle.within_tolerance(good, y, S)
    assert ok.all()
    # an error of 2^-7 |y| + 2^-11 S exceeds the bound everywhere it is nonzero
    bad_vals = y + np.sign(y + 0.5) * (2.0 ** -7 * np.abs(y) + 2.0 ** -11 * S)
    bad = np.array([[oracle.bf16_from_f64(v) for v in bad_vals[0]]], np.uint16)
    ok, _ = oracle.within_tolerance(bad, y, S)
    assert not ok.any()
    inf = np.array([[0x7F80, 0x7FC0, 0xFF80, 0x7F80]], np.uint16)
    ok, _ = oracle.within_tolerance(inf, y, S)
    assert not ok.any()


def test_a_bf16_rounded_output_always_passes_the_bound():
    # the exact result rounded once to bf16 lies within half an ulp of y, i.e.
    # within 2^-8 |y| (the worst case is just above a power of two)
    rng = np.random.default_rng(18)
    y = rng.standard_normal((1, 2000)) * 10.0 ** rng.integers(-5, 5, (1, 2000))
    out = np.array([[oracle.bf16_from_f64(v) for v in y[0]]], np.uint16)
    ok, ex = oracle.within_tolerance(out, y, np.zeros_like(y))
    assert ok.all() and ex.max() <= 1.0


def test_the_bound_reaches_down_to_bf16_subnormals():
    # below bf16's normal range (2^-126) its values are spaced 2^-133 apart:
    # the correctly rounded result of a y there can be 2^-134 away (more than
    # 2^-8 |y|), and it still passes; the floor adds nothing a normal-range
    # check would notice, and an error of two steps fails
    rng = np.random.default_rng(19)
    y = np.concatenate([rng.uniform(-1, 1, 400) * 2.0 ** -126, rng.uniform(-1, 1, 400) * 2.0 ** -134,
                        [2.0 ** -134, 3 * 2.0 ** -134, -2.0 ** -130, 2.0 ** -120]])[None, :]
    out = np.array([[oracle.bf16_from_f64(v) for v in y[0]]], np.uint16)
    S = np.zeros_like(y)
    ok, ex = oracle.within_tolerance(out, y, S)
    assert ok.all() and ex.max() <= 1.0
    assert np.any(np.abs(oracle.bf16_to_f64(out) - y) > 2.0 ** -8 * np.abs(y))   # the floor is what passes these
    off = np.array([[oracle.bf16_from_f64(v + np.copysign(2.0 * 2.0 ** -133, v)) for v in y[0]]], np.uint16)
    ok, _ = oracle.within_tolerance(off, y, S)
    assert not ok[0, :800].any()
