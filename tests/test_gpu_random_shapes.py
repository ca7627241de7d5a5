"""Seeded random shapes through the planner's routes: the decode-width
kernel, 128-row and 256-row tiles, the few-token instantiations with their
K split, both FP8 scale forms and NVFP4, all three epilogues (the tails of
products larger than one round are covered by the sampled full-size tests).
Whole outputs are compared with the oracle (quantize -> exact GEMM sums ->
scales -> epilogue) within the acceptance bound; the quantized codes and
scales must match bit for bit.  The shapes are drawn once from a fixed
seed, small enough for the oracle to finish in a few seconds each.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_normal

pytestmark = pytest.mark.gpu


def _cases(n=72, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fmt = ("e4m3_row", "e4m3_tensor", "nvfp4")[i % 3]
        epi = ("store", "add", "swiglu")[(i // 3) % 3]
        M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 129)), int(rng.integers(129, 520))]))
        N = int(rng.integers(1, 500)) * 2
        kq = 32 if fmt == "nvfp4" else 16
        K = int(rng.integers(1, 1600 // kq + 1)) * kq
        out.append((fmt, epi, M, N, K))
    # shapes that reach the few-token K split, 256-row tiles, and 128-row
    # tiles over several raster groups
    out += [("e4m3_row", "add", 40, 1024, 8192), ("nvfp4", "store", 48, 2048, 4096),
            ("e4m3_row", "add", 512, 16640, 256), ("e4m3_tensor", "store", 512, 16640, 512),
            ("e4m3_row", "store", 1300, 2560, 512), ("e4m3_tensor", "swiglu", 700, 4352, 512)]
    return out


CASES = _cases()


def dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def spg():
    import scaled_precision_gemm_amd as m
    return m


@pytest.mark.parametrize("fmt,epi,M,N,K", CASES, ids=lambda v: str(v))
def test_random_shape_matches_the_oracle(spg, fmt, epi, M, N, K):
    plan = spg.gemm_plan(M, N, K, fmt, epi)
    print(f"{fmt} {epi} {M}x{N}x{K} kernel {plan['kernel']} split {plan['split_k']} "
          f"tail {plan['tail_tiles']}/{plan['tail_split']}/{plan['tail_bm']}", flush=True)
    n_out = N // 2 if epi == "swiglu" else N
    A16 = bf16_normal((M, K), 1.0, 7 * M + K)
    W16 = bf16_normal((N, K), 0.02 if fmt != "e4m3_tensor" else 1.0, 11 * N + K)
    R16 = bf16_normal((M, n_out), 1.0, M + N) if epi == "add" else None
    res = dev(R16) if R16 is not None else None
    A, W = dev(A16), dev(W16)
    if fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        qa_o, sa_o = oracle.quantize_rowwise(A16)
        qw_o, sw_o = oracle.quantize_rowwise(W16)
        assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(sa.cpu().numpy(), sa_o)
        assert np.array_equal(qw.cpu().numpy(), qw_o) and np.array_equal(sw.cpu().numpy(), sw_o)
        out = spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res)
        D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        y, S, _ = oracle.epilogue(epi, D, Da, sa_o, sw_o, R16)
    elif fmt == "e4m3_tensor":
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        qa_o, sa_o = oracle.quantize_tensor(A16)
        qw_o, sw_o = oracle.quantize_tensor(W16)
        assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(sa.cpu().numpy(), sa_o)
        assert np.array_equal(qw.cpu().numpy(), qw_o) and np.array_equal(sw.cpu().numpy(), sw_o)
        out = spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res, fmt="e4m3_tensor")
        D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        y, S, _ = oracle.epilogue(epi, D, Da, sa_o[0], sw_o[0], R16)
    else:
        qa, ba, ta = spg.quantize_block16(A)
        qw, bw, tw = spg.quantize_block16(W)
        qa_o, ba_o, ta_o = oracle.quantize_block16(A16)
        qw_o, bw_o, tw_o = oracle.quantize_block16(W16)
        assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(ba.cpu().numpy(), ba_o)
        assert np.array_equal(qw.cpu().numpy(), qw_o) and np.array_equal(bw.cpu().numpy(), bw_o)
        assert ta.cpu().numpy()[0] == ta_o and tw.cpu().numpy()[0] == tw_o
        out = spg.gemm_scaled(qa, ba, qw, bw, epi, residual=res, fmt="nvfp4", tscale_a=ta, tscale_w=tw)
        D, Da = oracle.gemm_nvfp4_sums(qa_o, ba_o, qw_o, bw_o)
        y, S, _ = oracle.epilogue(epi, D, Da, ta_o, tw_o, R16)
    got = host(out)
    assert got.shape == (M, n_out)
    ok, excess = oracle.within_tolerance(got, y, S)
    bad = np.argwhere(~ok)
    assert ok.all(), f"{len(bad)} of {ok.size} outside the bound; worst excess {excess.max():.3g} at {bad[:5].tolist()}"


# Rows of A and W scaled by random powers of ten (A: 1e-30 .. 1e30, W:
# 1e-20 .. 1e20; SwiGLU, whose epilogue forms gate x up in fp32 first:
# 1e-10 .. 1e10 and 1e-5 .. 1e5), so the row scales, their products and the
# outputs span most of the fp32 and bf16 range, subnormal-scale rows included.
WIDE = [(int(m), int(n) * 2, int(k) * 16, epi) for m, n, k, epi in
        zip(np.random.default_rng(77).integers(1, 400, 12), np.random.default_rng(78).integers(1, 300, 12),
            np.random.default_rng(79).integers(1, 80, 12), ["store", "add", "swiglu"] * 4)]
# Shapes whose data (seeded by the shape) hold a gate sum that cancels to
# ~1e-6 of its sum of |products|, so that the fp32 gate is off by far more
# than silu's slope at the exact gate allows (gates -13.6, -767 and -1.1e8),
# and a sum that cancels to exactly zero under a row-scale product beyond
# fp32's range.
WIDE += [(99, 770, 1408, "swiglu"), (489, 326, 1568, "swiglu"), (329, 208, 1600, "swiglu"), (671, 406, 96, "store")]
# and shapes the planner splits along K (the reduction applies the epilogue)
WIDE += [(48, 1024, 4096, "add"), (200, 600, 3072, "swiglu"), (40, 900, 6144, "store")]


@pytest.mark.parametrize("M,N,K,epi", WIDE, ids=lambda v: str(v))
def test_row_scales_across_the_range_match_the_oracle(spg, M, N, K, epi):
    rng = np.random.default_rng(M * N + K)
    from synthetic import f32_to_bf16_bits
    ea, ew = (10, 5) if epi == "swiglu" else (30, 20)
    fa = oracle.bf16_to_f64(bf16_normal((M, K), 1.0, M + 5)) * 10.0 ** rng.uniform(-ea, ea, (M, 1))
    fw = oracle.bf16_to_f64(bf16_normal((N, K), 1.0, N + 6)) * 10.0 ** rng.uniform(-ew, ew, (N, 1))
    A16 = f32_to_bf16_bits(fa.astype(np.float32))
    W16 = f32_to_bf16_bits(fw.astype(np.float32))
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, M + N) if epi == "add" else None
    qa, sa = spg.quantize_rowwise(dev(A16))
    qw, sw = spg.quantize_rowwise(dev(W16))
    qa_o, sa_o = oracle.quantize_rowwise(A16)
    qw_o, sw_o = oracle.quantize_rowwise(W16)
    assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(sa.cpu().numpy(), sa_o)
    assert np.array_equal(qw.cpu().numpy(), qw_o) and np.array_equal(sw.cpu().numpy(), sw_o)
    got = host(spg.gemm_scaled(qa, sa, qw, sw, epi, residual=dev(R16) if R16 is not None else None))
    D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
    y, S, _ = oracle.epilogue(epi, D, Da, sa_o, sw_o, R16)
    # elements whose acceptance interval reaches beyond bf16's finite range
    # are not compared (there a sum that cancels to zero exactly may come out
    # as a small fp32 residue times a scale product beyond fp32's range)
    fin = np.isfinite(y) & (np.abs(y) + 2.0 ** -12 * S < 3.0e38)
    ok, excess = oracle.within_tolerance(got, y, S)
    bad = np.argwhere(fin & ~ok)
    assert len(bad) == 0, f"{len(bad)} outside the bound; worst excess {excess[fin].max():.3g} at {bad[:5].tolist()}"


@pytest.mark.parametrize("epi", ["store", "add"])
def test_nvfp4_tensor_scales_whose_product_passes_fp32_range(spg, epi):
    # A holds one element of 4e28 (column 0) and W one of 4e12 (column 16,
    # another K block), the rest ~1e25 and ~1e9: 2^14 tA tW is beyond fp32's
    # range while every output (~1e38) is finite in bf16, so the tensor
    # scales must not be folded into one fp32 factor
    M, N, K = 8, 90, 704
    fa = oracle.bf16_to_f64(bf16_normal((M, K), 1.0, 31)) * 1e25
    fw = oracle.bf16_to_f64(bf16_normal((N, K), 1.0, 32)) * 1e9
    fa[:, 0] = 4e28
    fw[:, 16] = 4e12
    from synthetic import f32_to_bf16_bits
    A16 = f32_to_bf16_bits(fa.astype(np.float32))
    W16 = f32_to_bf16_bits(fw.astype(np.float32))
    R16 = bf16_normal((M, N), 1.0, 33) if epi == "add" else None
    qa, ba, ta = spg.quantize_block16(dev(A16))
    qw, bw, tw = spg.quantize_block16(dev(W16))
    qa_o, ba_o, ta_o = oracle.quantize_block16(A16)
    qw_o, bw_o, tw_o = oracle.quantize_block16(W16)
    assert np.array_equal(qa.cpu().numpy(), qa_o) and np.array_equal(qw.cpu().numpy(), qw_o)
    assert ta.cpu().numpy()[0] == ta_o and tw.cpu().numpy()[0] == tw_o
    assert 16384.0 * float(ta_o) * float(tw_o) > 3.5e38      # the folded factor would be inf in fp32
    got = host(spg.gemm_scaled(qa, ba, qw, bw, epi, residual=dev(R16) if R16 is not None else None, fmt="nvfp4",
                               tscale_a=ta, tscale_w=tw))
    D, Da = oracle.gemm_nvfp4_sums(qa_o, ba_o, qw_o, bw_o)
    y, S, _ = oracle.epilogue(epi, D, Da, ta_o, tw_o, R16)
    assert np.all(np.abs(y) + 2.0 ** -12 * S < 3.0e38) and np.abs(y).max() > 1e37
    ok, excess = oracle.within_tolerance(got, y, S)
    bad = np.argwhere(~ok)
    assert ok.all(), f"{len(bad)} outside the bound; worst excess {excess.max():.3g} at {bad[:5].tolist()}"
