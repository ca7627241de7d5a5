"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Quantizers must match bit for bit (codes and fp32 scales).  GEMM outputs must
satisfy, per element, |gpu - y| <= 2^-8 |y| + 2^-12 S, with y the oracle's
exact fp64 result and S the scaled sum of |products|.  The oracle quantizes
the bf16 inputs itself: no oracle input comes from the GPU.  Full-size
workloads are checked on sampled rows x columns (tile edges included).
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from synthetic import WORKLOADS, bf16_normal, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import scaled_precision_gemm_amd as m
    return m


def dev(x16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).view(torch.bfloat16).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_close(gpu_bits, y, S, what):
    ok, excess = oracle.within_tolerance(gpu_bits, y, S)
    bad = np.argwhere(~ok)
    assert ok.all(), (f"{what}: {len(bad)} of {ok.size} outside the bound; worst excess {excess.max():.3g} "
                      f"at {bad[:5].tolist()}")


# ---------------------------------------------------------------------------
# quantize_rowwise
# ---------------------------------------------------------------------------
ROW_SHAPES = [(1, 16), (17, 48), (321, 512), (5, 1024), (3, 1040), (9, 2048), (4, 4096), (5, 5136), (6, 8192), (3, 12288),
              (2, 16384), (7, 17408), (3, 40000)]


@pytest.mark.parametrize("shape", ROW_SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_quantize_rowwise_bitexact(spg, shape):
    x = bf16_normal(shape, 1.0, 1000 + shape[1])
    q, s = spg.quantize_rowwise(dev(x))
    qo, so = oracle.quantize_rowwise(x)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("name", ["fp8_row_tiny", "fp8_row_add_t1024", "fp8_row_swiglu_t4096"])
def test_quantize_rowwise_bitexact_workloads(spg, name):
    wl = WORKLOADS[name]
    A, W, _ = wl.inputs()
    for x in (A, W):
        q, s = spg.quantize_rowwise(dev(x))
        qo, so = oracle.quantize_rowwise(x)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        assert np.array_equal(q.cpu().numpy(), qo)
        del q, s


def test_quantize_rowwise_every_bf16_value_with_unit_and_pow2_scales(spg):
    # rows led by 448 * 2^k have scale exactly 2^k, so every bf16 value of
    # magnitude <= 448 * 2^k is encoded directly: all roundings and ties
    u = np.arange(65536, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    for k in (0, -7, 5):
        top = np.float32(448.0 * 2.0 ** k)
        vals = f[np.isfinite(f) & (np.abs(f) <= top)]
        K = 4096
        n = (len(vals) + K - 2) // (K - 1)
        body = np.resize(vals, n * (K - 1)).reshape(n, K - 1)
        x = np.concatenate([np.full((n, 1), top, np.float32), body], axis=1)
        x16 = f32_to_bf16_bits(x)
        q, s = spg.quantize_rowwise(dev(x16))
        qo, so = oracle.quantize_rowwise(x16)
        assert np.all(so == np.float32(2.0 ** k))
        assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
        assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("K", [256, 2064], ids=["one_wave_per_row", "one_block_per_row"])
def test_quantize_rowwise_every_amax_exponent(spg, K):
    # one row per amax: every bf16 exponent (subnormal amax included), both
    # sides of 2^-40 and the largest finite bf16; the rest of each row is
    # random bit patterns of magnitude <= amax with random signs, so values
    # of every size down to subnormals meet a scale of every size (K = 2064:
    # rows for the four-wave kernel, with a partly filled last vector column)
    rng = np.random.default_rng(77)
    amax = [(e << 7) | int(rng.integers(0, 128)) for e in range(0, 255)]
    amax += [0x0001, 0x007F, 0x0080, 0x2B7F, 0x2B80, 0x2B81, 0x7F7F]
    x = np.zeros((len(amax), K), np.uint16)
    for i, a in enumerate(amax):
        body = rng.integers(0, a + 1, size=K - 1).astype(np.uint16)
        body |= (rng.integers(0, 2, size=K - 1) << 15).astype(np.uint16)
        x[i, 0] = a
        x[i, 1:] = body
    q, s = spg.quantize_rowwise(dev(x))
    qo, so = oracle.quantize_rowwise(x)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)
    # the per-tensor quantizer takes the same path with one scale per matrix
    for i in (0, 3, 100, 200, len(amax) - 1):
        qt, st = spg.quantize_tensor(dev(x[i:i + 1]))
        qto, sto = oracle.quantize_tensor(x[i:i + 1])
        assert np.array_equal(st.cpu().numpy().view(np.uint32), sto.view(np.uint32))
        assert np.array_equal(qt.cpu().numpy(), qto)


def _every_amax_rows(a_lo, a_hi):
    """Rows [amax, every bf16 x with |x| <= amax] for the positive finite
    bf16 amax patterns a_lo .. a_hi - 1 (positive bf16 bit patterns order as
    their values), zero-padded to a common multiple of 16."""
    a = np.arange(a_lo, a_hi, dtype=np.int32)[:, None]
    K = int(-(-(2 * (a_hi - 1) + 3) // 16) * 16)
    i = np.arange(K, dtype=np.int32)[None, :]
    x = np.where(i == 0, a, 0)
    x = np.where((i >= 1) & (i <= a + 1), i - 1, x)
    x = np.where((i >= a + 2) & (i <= 2 * a + 2), 0x8000 | (i - a - 2), x)
    return x.astype(np.uint16)


# chunk boundaries over the 32639 positive finite bf16 amax patterns, spaced
# so each chunk holds about the same number of (amax, x) pairs
_AMAX_EDGES = [1] + [int(0x7F80 * np.sqrt(k / 8.0)) for k in range(1, 8)] + [0x7F80]


@pytest.mark.parametrize("chunk", range(8))
def test_quantize_rowwise_every_amax_times_every_x(spg, chunk):
    # exhaustive over the division-free encoder: every positive finite bf16
    # amax (so every scale the row-wise quantizer can form, subnormal ones
    # and the 2^100-scaled path for amax < 2^-40 included) against every bf16
    # value x with |x| <= amax, both signs; codes and scales bit for bit
    a_lo, a_hi = _AMAX_EDGES[chunk], _AMAX_EDGES[chunk + 1]
    print(f"amax patterns {a_lo:#06x} .. {a_hi - 1:#06x}", flush=True)
    x = _every_amax_rows(a_lo, a_hi)
    q, s = spg.quantize_rowwise(dev(x))
    qo, so = oracle.quantize_rowwise(x)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    qg = q.cpu().numpy()
    bad = np.argwhere(qg != qo)
    assert len(bad) == 0, (f"{len(bad)} codes differ, first (row amax, x): "
                           f"{[(int(x[r, 0]), int(x[r, c])) for r, c in bad[:5]]}")
    del q, s
    torch.cuda.empty_cache()


def test_quantize_rowwise_zero_and_signed_zero_rows(spg):
    x = np.zeros((3, 64), np.uint16)
    x[1, ::3] = 0x8000
    x[2] = bf16_normal((64,), 1.0, 5)
    q, s = spg.quantize_rowwise(dev(x))
    qo, so = oracle.quantize_rowwise(x)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)


def test_quantize_rowwise_strided_rows(spg):
    x = bf16_normal((40, 160), 1.0, 6)
    xt = dev(x)[:, :128]                       # row stride 160, K 128
    q = torch.full((40, 144), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.empty(40, dtype=torch.float32, device="cuda")
    spg.quantize_rowwise(xt, out=q[:, :128], scale=s)
    qo, so = oracle.quantize_rowwise(np.ascontiguousarray(x[:, :128]))
    qh = q.cpu().numpy()
    assert np.array_equal(qh[:, :128], qo) and np.all(qh[:, 128:] == 0xAB)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))


# ---------------------------------------------------------------------------
# quantize_tensor / quantize_block16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 5, 32), (3, 17, 48), (64, 512, 512), (1, 8192, 8192)],
                         ids=lambda s: "x".join(map(str, s)))
def test_quantize_tensor_bitexact(spg, shape):
    x = bf16_normal(shape, 1.0, 2000 + shape[0])
    q, s = spg.quantize_tensor(dev(x))
    qo, so = oracle.quantize_tensor(x)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), qo)


@pytest.mark.parametrize("shape,std", [((1, 32), 1.0), ((7, 64), 1.0), ((33, 96), 0.02), ((4096, 6144), 1.0),
                                       ((5120, 6144), 0.02)], ids=lambda v: str(v))
def test_quantize_block16_bitexact(spg, shape, std):
    x = bf16_normal(shape, std, 3000 + shape[0])
    q, bs, t = spg.quantize_block16(dev(x))
    qo, bso, to = oracle.quantize_block16(x)
    assert t.cpu().numpy().view(np.uint32)[0] == np.float32(to).view(np.uint32)
    assert np.array_equal(bs.cpu().numpy(), bso)
    assert np.array_equal(q.cpu().numpy(), qo)


def unblock_scales(plane: np.ndarray, R: int, K: int) -> np.ndarray:
    """Row-major [R, K/16] view of a blocked NVFP4 scale plane (4 KiB blocks
    of 256 rows x 16 scale bytes, by row tile then K stage) and its padding
    rows."""
    tiles, stages = plane.shape[0], plane.shape[1]
    full = plane.reshape(tiles, stages, 256, 16).transpose(0, 2, 1, 3).reshape(tiles * 256, stages * 16)
    return full[:R], full[R:]


@pytest.mark.parametrize("shape,std", [((1, 256), 1.0), ((300, 512), 1.0), ((257, 1024), 0.02), ((4096, 6144), 1.0),
                                       ((5120, 6144), 0.02), ((6144, 8448), 1.0)], ids=lambda v: str(v))
def test_quantize_block16_blocked_layout(spg, shape, std):
    # the blocked plane holds exactly the row-major scales, padding rows are
    # zero, and codes and the tensor scale do not depend on the layout; the
    # last shape is beyond one resident grid (the two-pass path)
    R, K = shape
    x16 = bf16_normal(shape, std, 3100 + R)
    path = spg.lib.quantize_block16_path(R, K)
    assert path == (2 if R * K > 40_000_000 else 1)
    x = dev(x16)
    qo, bso, to = oracle.quantize_block16(x16)
    for single in (False, True):         # two passes; single launch where the tensor fits one grid
        q, bs, t = spg.quantize_block16(x, layout="blocked", single_launch=single)
        qr, bsr, tr = spg.quantize_block16(x, layout="row", single_launch=single)
        plane, pad = unblock_scales(bs.cpu().numpy(), R, K)
        assert t.cpu().numpy().view(np.uint32)[0] == np.float32(to).view(np.uint32) == tr.cpu().numpy().view(np.uint32)[0]
        assert np.array_equal(plane, bso) and np.array_equal(bsr.cpu().numpy(), bso)
        assert pad.size == ((-R) % 256) * (K // 16) and np.all(pad == 0)
        assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(qr.cpu().numpy(), qo)


def test_quantize_block16_every_bf16_value_in_unit_groups(spg):
    # tensor amax 2688 gives t = 1; a group led by 6 gets scale code 1.0,
    # so its other 15 values are encoded directly to E2M1
    u = np.arange(65536, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    vals = f[np.isfinite(f) & (np.abs(f) <= 6.0)]
    n = (len(vals) + 14) // 15
    body = np.resize(vals, n * 15).reshape(n, 15)
    groups = np.concatenate([np.full((n, 1), 6.0, np.float32), body], axis=1)
    K = 256
    rows = (n + K // 16 - 1) // (K // 16)
    pad = rows * (K // 16) - n
    groups = np.concatenate([groups, np.tile(groups[:1], (pad, 1))])
    x = groups.reshape(rows, K)
    x[0, 0] = 2688.0
    x16 = f32_to_bf16_bits(x)
    q, bs, t = spg.quantize_block16(dev(x16))
    qo, bso, to = oracle.quantize_block16(x16)
    assert to == 1.0
    assert np.array_equal(bs.cpu().numpy(), bso)
    assert np.array_equal(q.cpu().numpy(), qo)


def test_fp4_conversion_instruction_matches_the_e2m1_encoder(spg):
    # the NVFP4 quantizers round with v_cvt_scalef32_pk_fp4_f32: it must give
    # the library's E2M1 code (nearest even, saturating, signed zero) for
    # every binary32 input that is not a NaN
    r = spg.probe_fp4_rounding()
    assert r["differences"] == 0, r["examples"]


def test_quantize_block16_wide_scale_range_and_zero(spg):
    # group magnitudes from 2^-20 to 1 relative to the tensor maximum:
    # subnormal and zero block-scale codes
    x = bf16_normal((16, 512), 1.0, 7).astype(np.uint32)
    xf = (x << 16).view(np.float32).reshape(16, 32, 16)
    xf *= (2.0 ** -np.linspace(0, 20, 32, dtype=np.float32))[None, :, None]
    xf[3] = 0.0
    x16 = f32_to_bf16_bits(xf.reshape(16, 512))
    q, bs, t = spg.quantize_block16(dev(x16))
    qo, bso, to = oracle.quantize_block16(x16)
    assert np.array_equal(bs.cpu().numpy(), bso) and np.any(bso < 8) and np.any(bso == 0)
    assert np.array_equal(q.cpu().numpy(), qo)


# ---------------------------------------------------------------------------
# GEMM, whole outputs (small and ragged shapes)
# ---------------------------------------------------------------------------

def run_fp8(spg, A16, W16, epi, fmt, R16=None):
    A, W = dev(A16), dev(W16)
    if fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
    else:
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
    out = spg.gemm_scaled(qa, sa, qw, sw, epi, residual=dev(R16) if R16 is not None else None, fmt=fmt)
    return host_u16(out)


def oracle_fp8(A16, W16, epi, fmt, R16=None):
    if fmt == "e4m3_row":
        return oracle.linear_e4m3_rowwise(A16, W16, epi, R16)
    qa, sa = oracle.quantize_tensor(A16)
    qw, sw = oracle.quantize_tensor(W16)
    D, Da = oracle.gemm_e4m3_sums(qa, qw)
    y, S, out = oracle.epilogue(epi, D, Da, sa[0], sw[0], R16)
    return dict(y=y, S=S, out=out)


SMALL = [(128, 256, 512), (1, 2, 16), (17, 34, 48), (257, 300, 160), (300, 258, 1040), (64, 512, 384)]


@pytest.mark.parametrize("fmt", ["e4m3_row", "e4m3_tensor"])
@pytest.mark.parametrize("epi", ["store", "add", "swiglu"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_gemm_fp8_small_shapes(spg, shape, epi, fmt):
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, M * 7 + K)
    W16 = bf16_normal((N, K), 0.02, N * 11 + K)
    R16 = bf16_normal((M, N), 1.0, M + N) if epi == "add" else None
    gpu = run_fp8(spg, A16, W16, epi, fmt, R16)
    ref = oracle_fp8(A16, W16, epi, fmt, R16)
    assert gpu.shape == ref["out"].shape
    check_close(gpu, ref["y"], ref["S"], f"{shape} {epi} {fmt}")


def test_bound_rejects_planted_errors_on_a_gpu_output(spg):
    # the acceptance check is not vacuous on real data: the 128 x 256 x 512
    # store output of the GPU passes it, and the same output moved away from
    # y by 2^-7 |y| + 2^-11 S (twice the bound) fails it wherever the bound
    # is nonzero
    wl = WORKLOADS["fp8_row_tiny"]
    A16, W16, _ = wl.inputs()
    gpu = run_fp8(spg, A16, W16, "store", "e4m3_row", None)
    ref = oracle_fp8(A16, W16, "store", "e4m3_row", None)
    check_close(gpu, ref["y"], ref["S"], "tiny store")
    g = oracle.bf16_to_f64(gpu)
    away = np.where(g >= ref["y"], 1.0, -1.0)
    planted = g + away * (2.0 ** -7 * np.abs(ref["y"]) + 2.0 ** -11 * ref["S"])
    bad = np.vectorize(oracle.bf16_from_f64, otypes=[np.uint16])(planted)
    ok, _ = oracle.within_tolerance(bad, ref["y"], ref["S"])
    assert not ok.any()
    with pytest.raises(AssertionError):
        check_close(bad, ref["y"], ref["S"], "planted")


# extreme aspect ratios: many tiles along one dimension (more tiles than
# compute units, so the persistent grid walks several per workgroup), and the
# longest K the oracle's fp64 sums keep exact (2^16; split 8 ways along K).
# 513 x 65792 x 256 SWIGLU: 771 tiles of two K stages on the persistent
# grid, three or four per workgroup, so every buffer of the row-wise SWIGLU
# scale ring is used (and a last tile row of one token), checked in full.
EXTREME = [((70000, 40, 256), "add"), ((3, 70000, 256), "store"), ((5, 80000, 64), "swiglu"),
           ((513, 65792, 256), "swiglu"), ((40, 72, 65536), "store"), ((130, 264, 65536), "swiglu")]


@pytest.mark.parametrize("shape,epi", EXTREME, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_gemm_fp8_extreme_shapes(spg, shape, epi):
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, M + 3 * K)
    W16 = bf16_normal((N, K), 0.02, N + 5 * K)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, M + N + 1) if epi == "add" else None
    gpu = run_fp8(spg, A16, W16, epi, "e4m3_row", R16)
    ref = oracle_fp8(A16, W16, epi, "e4m3_row", R16)
    assert gpu.shape == ref["out"].shape
    check_close(gpu, ref["y"], ref["S"], f"{shape} {epi}")


@pytest.mark.parametrize("M,N,K,kernel", [(300, 260, 256, 2), (4096, 5120, 2048, 0)],
                         ids=["half_tiles", "persistent_with_half_tail"])
def test_gemm_zero_weight_add_returns_residual_bitwise(spg, M, N, K, kernel):
    # every residual element lands where it belongs: whole-quadrant passes
    # (each pass's residual loaded during the pass before), staged blocks of
    # the half-height kernel, ragged edges
    assert spg.gemm_plan(M, N, K, "e4m3_row", "add")["kernel"] == kernel
    A16 = bf16_normal((M, K), 1.0, 1)
    W16 = np.zeros((N, K), np.uint16)
    R16 = bf16_normal((M, N), 1.0, 2)
    gpu = run_fp8(spg, A16, W16, "add", "e4m3_row", R16)
    # the product is +0, and +0 + r is r except for r = -0 (IEEE: +0)
    assert np.any(R16 == 0x8000) == (kernel == 0)   # this residual holds one -0
    assert np.array_equal(gpu, np.where(R16 == 0x8000, np.uint16(0), R16))


@pytest.mark.parametrize("fmt", ["e4m3_row", "e4m3_tensor"])
@pytest.mark.parametrize("epi", ["store", "add", "swiglu"])
def test_gemm_empty_k(spg, epi, fmt):
    # K = 0 through the C ABI (the binding cannot pass the null data pointer
    # of an empty torch tensor): every sum is empty, so the output is exactly
    # zero (SWIGLU: silu(0) * 0) or the residual, bit for bit.  600 tiles:
    # the persistent grid walks up to three per workgroup with no K stages
    # between them.
    M, N = 300, 76800
    n_out = N // 2 if epi == "swiglu" else N
    A = torch.zeros((M, 16), dtype=torch.uint8, device="cuda")
    W = torch.zeros((N, 16), dtype=torch.uint8, device="cuda")
    nsc = (M, N) if fmt == "e4m3_row" else (1, 1)
    sa = torch.full((nsc[0],), 0.75, dtype=torch.float32, device="cuda")
    sw = torch.full((nsc[1],), 1.5, dtype=torch.float32, device="cuda")
    R16 = bf16_normal((M, n_out), 1.0, 41) if epi == "add" else None
    res = dev(R16) if R16 is not None else None
    out = torch.full((M, n_out), -1.0, dtype=torch.bfloat16, device="cuda")
    d, e, _ = spg.make_desc(A, W, fmt, epi, out, res)
    d.K = 0
    assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), e) == 0
    st = spg.lib.gemm_scaled(out.data_ptr(), A.data_ptr(), sa.data_ptr(), W.data_ptr(), sw.data_ptr(),
                             res.data_ptr() if res is not None else None, e, ctypes.byref(d), None, 0,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0
    gpu = host_u16(out)
    assert np.array_equal(gpu, R16 if epi == "add" else np.zeros((M, n_out), np.uint16))


def test_gemm_power_of_two_case_is_bitwise(spg):
    # codes from a narrow exponent band with power-of-two scales: every partial
    # sum is exact in fp32 whatever the order, so the GPU output must equal
    # the oracle's single rounding bit for bit
    rng = np.random.default_rng(3)
    M, N, K = 96, 160, 64
    vals = np.array([1.0, 1.125, 1.25, 1.5, 1.75, 2.0, -1.0, -1.5, -2.0, 0.0], np.float32)
    A = rng.choice(vals, (M, K)).astype(np.float32)
    W = rng.choice(vals, (N, K)).astype(np.float32) * np.float32(2.0 ** -3)
    A[:, 0] = 448.0 * 2.0 ** -4
    W[:, 0] = 448.0 * 2.0 ** -9
    A16, W16 = f32_to_bf16_bits(A), f32_to_bf16_bits(W)
    gpu = run_fp8(spg, A16, W16, "store", "e4m3_row")
    ref = oracle.linear_e4m3_rowwise(A16, W16, "store")
    assert np.all(ref["sa"] == np.float32(2.0 ** -4)) and np.all(ref["sw"] == np.float32(2.0 ** -9))
    assert np.array_equal(gpu, ref["out"])


def test_gemm_batched_tensor_scale_with_broadcast_weight(spg):
    B, M, N, K = 3, 100, 72, 96
    A16 = bf16_normal((B, M, K), 1.0, 9)
    W16 = bf16_normal((N, K), 1.0, 10)
    qa, sa = spg.quantize_tensor(dev(A16))
    qw, sw = spg.quantize_tensor(dev(W16))
    out = host_u16(spg.gemm_scaled(qa, sa, qw, sw, "store", fmt="e4m3_tensor"))
    qwo, swo = oracle.quantize_tensor(W16)
    for b in range(B):
        qao, sao = oracle.quantize_tensor(A16[b])
        D, Da = oracle.gemm_e4m3_sums(qao, qwo)
        y, S, _ = oracle.epilogue("store", D, Da, sao[0], swo[0])
        check_close(out[b], y, S, f"batch {b}")


def test_gemm_add_in_place(spg):
    M, N, K = 130, 260, 128
    A16 = bf16_normal((M, K), 1.0, 21)
    W16 = bf16_normal((N, K), 0.02, 22)
    R16 = bf16_normal((M, N), 1.0, 23)
    qa, sa = spg.quantize_rowwise(dev(A16))
    qw, sw = spg.quantize_rowwise(dev(W16))
    r = dev(R16)
    spg.gemm_scaled(qa, sa, qw, sw, "add", residual=r, out=r)
    ref = oracle.linear_e4m3_rowwise(A16, W16, "add", R16)
    check_close(host_u16(r), ref["y"], ref["S"], "in-place add")


def test_binding_cache_rechecks_changed_signatures(spg):
    # gemm_scaled reuses the checked descriptor of a repeated call signature
    # (shapes, strides, dtypes, devices, pointer alignment); any change of
    # those is checked again
    M, N, K = 16, 512, 256
    A16 = bf16_normal((M, K), 1.0, 41)
    W16 = bf16_normal((N, K), 0.02, 42)
    qa, sa = spg.quantize_rowwise(dev(A16))
    qw, sw = spg.quantize_rowwise(dev(W16))
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    r1 = spg.gemm_scaled(qa, sa, qw, sw, out=out).clone()
    r2 = spg.gemm_scaled(qa, sa, qw, sw, out=out)             # the cached descriptor
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    with pytest.raises(ValueError):
        spg.gemm_scaled(qa, sa, qw, sw, out=torch.empty((M, N + 8), dtype=torch.bfloat16, device="cuda"))
    # K-major W: 16-byte aligned rows pass; the same shape one byte off does not
    wt = torch.zeros((K, N + 16), dtype=torch.uint8, device="cuda")
    wt[:, :N] = qw.t()
    for _ in range(2):
        rk = spg.gemm_scaled(qa, sa, wt[:, :N], sw, w_kmajor=True)
        assert torch.equal(rk.view(torch.int16), r1.view(torch.int16))
    with pytest.raises(ValueError, match="16-byte"):
        spg.gemm_scaled(qa, sa, wt[:, 1:N + 1], sw, w_kmajor=True)
    ref = oracle_fp8(A16, W16, "store", "e4m3_row", None)
    check_close(host_u16(r1), ref["y"], ref["S"], "cached call")


def test_gemm_is_deterministic(spg):
    A16 = bf16_normal((1024, 2048), 1.0, 31)
    W16 = bf16_normal((512, 2048), 0.02, 32)
    R16 = bf16_normal((1024, 512), 1.0, 33)
    a = run_fp8(spg, A16, W16, "add", "e4m3_row", R16)
    b = run_fp8(spg, A16, W16, "add", "e4m3_row", R16)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# NVFP4
# ---------------------------------------------------------------------------

def run_nvfp4(spg, A16, W16, epi, R16=None):
    qa, bsa, ta = spg.quantize_block16(dev(A16))
    qw, bsw, tw = spg.quantize_block16(dev(W16))
    out = spg.gemm_scaled(qa, bsa, qw, bsw, epi, residual=dev(R16) if R16 is not None else None,
                          fmt="nvfp4", tscale_a=ta, tscale_w=tw)
    return host_u16(out)


def oracle_nvfp4(A16, W16, epi, R16=None):
    qa, bsa, ta = oracle.quantize_block16(A16)
    qw, bsw, tw = oracle.quantize_block16(W16)
    D, Da = oracle.gemm_nvfp4_sums(qa, bsa, qw, bsw)
    y, S, out = oracle.epilogue(epi, D, Da, ta, tw, R16)
    return dict(y=y, S=S, out=out)


@pytest.mark.parametrize("epi", ["store", "add", "swiglu"])
@pytest.mark.parametrize("shape", [(64, 64, 64), (17, 40, 96), (257, 300, 320), (128, 512, 1056)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_nvfp4_small_shapes(spg, shape, epi):
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, 40 + M)
    W16 = bf16_normal((N, K), 0.02, 41 + N)
    R16 = bf16_normal((M, N), 1.0, 42) if epi == "add" else None
    gpu = run_nvfp4(spg, A16, W16, epi, R16)
    ref = oracle_nvfp4(A16, W16, epi, R16)
    check_close(gpu, ref["y"], ref["S"], f"nvfp4 {shape} {epi}")


# K a multiple of 256: the path that copies codes and scales straight into
# LDS (several tiles, ragged edges, and a single tile that the planner splits
# along K)
@pytest.mark.parametrize("epi", ["store", "add", "swiglu"])
@pytest.mark.parametrize("shape", [(64, 64, 256), (257, 300, 512), (300, 520, 1024), (256, 256, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_nvfp4_stage256_shapes(spg, shape, epi):
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, 60 + M)
    W16 = bf16_normal((N, K), 0.02, 61 + N)
    R16 = bf16_normal((M, N), 1.0, 62) if epi == "add" else None
    gpu = run_nvfp4(spg, A16, W16, epi, R16)
    ref = oracle_nvfp4(A16, W16, epi, R16)
    check_close(gpu, ref["y"], ref["S"], f"nvfp4 {shape} {epi}")


# blocked scale planes (K a multiple of 256): ragged M and N (zero padding
# rows), SwiGLU halves that are not multiples of 128 rows (up rows straddle
# the plane's 256-row blocks), and a single tile split along K
@pytest.mark.parametrize("epi", ["store", "add", "swiglu"])
@pytest.mark.parametrize("shape", [(64, 64, 256), (257, 400, 512), (300, 520, 1024), (256, 256, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
def test_gemm_nvfp4_blocked_scales(spg, shape, epi):
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, 160 + M)
    W16 = bf16_normal((N, K), 0.02, 161 + N)
    R16 = bf16_normal((M, N), 1.0, 162) if epi == "add" else None
    qa, bsa, ta = spg.quantize_block16(dev(A16), layout="blocked")
    qw, bsw, tw = spg.quantize_block16(dev(W16), layout="blocked")
    out = spg.gemm_scaled(qa, bsa, qw, bsw, epi, residual=dev(R16) if R16 is not None else None,
                          fmt="nvfp4", tscale_a=ta, tscale_w=tw, scale_layout="blocked")
    ref = oracle_nvfp4(A16, W16, epi, R16)
    check_close(host_u16(out), ref["y"], ref["S"], f"nvfp4 blocked {shape} {epi}")


def test_gemm_nvfp4_wide_scale_range(spg):
    # block scales spanning subnormal E4M3 codes exercise every decode path
    M, N, K = 96, 64, 512
    x = bf16_normal((M, K), 1.0, 50).astype(np.uint32)
    xf = (x << 16).view(np.float32).reshape(M, K // 16, 16)
    xf *= (2.0 ** -np.linspace(0, 18, K // 16, dtype=np.float32))[None, :, None]
    A16 = f32_to_bf16_bits(xf.reshape(M, K))
    W16 = bf16_normal((N, K), 0.02, 51)
    gpu = run_nvfp4(spg, A16, W16, "store")
    ref = oracle_nvfp4(A16, W16, "store")
    check_close(gpu, ref["y"], ref["S"], "nvfp4 wide scales")


# ---------------------------------------------------------------------------
# full-size workloads, sampled outputs
# ---------------------------------------------------------------------------

def sample(n, count, rng, tile=256):
    edges = [0, n - 1] + [v for t in range(tile, n, tile) for v in (t - 1, t)][:12]
    rest = rng.choice(n, size=max(0, count - len(edges)), replace=False)
    return np.unique(np.clip(np.concatenate([edges, rest]), 0, n - 1))


def sample_every_tile(n, rng, tile):
    """Indices 0 .. n-1 with two in every tile of `tile` indices, one in each
    half (so both 128-row halves of a half-height tile are hit), plus the
    first and last index and the edges of the first tiles."""
    picks = [0, n - 1] + [v for t in range(tile, n, tile) for v in (t - 1, t)][:8]
    half = tile // 2
    for t0 in range(0, n, tile):
        lo_end = min(t0 + half, n)
        picks.append(int(rng.integers(t0, lo_end)))
        if lo_end < n:
            picks.append(int(rng.integers(lo_end, min(t0 + tile, n))))
    return np.unique(np.asarray(picks, np.int64))


@pytest.mark.parametrize("name", ["fp8_row_add_t1024", "fp8_row_swiglu_t4096", "fp8_tensor_square_8192",
                                  "fp8_tensor_bmm64_512", "nvfp4_add_t4096", "fp8_row_bias_t4096"])
def test_workload_full_size_sampled(spg, name):
    wl = WORKLOADS[name]
    rng = np.random.default_rng(99)
    A16, W16, R16 = wl.inputs()
    A, W = dev(A16), dev(W16)
    R = dev(R16) if R16 is not None else None
    if wl.fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, wl.epilogue, residual=R)
    elif wl.fmt == "e4m3_tensor":
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, wl.epilogue, fmt="e4m3_tensor")
    else:
        qa, sa, ta = spg.quantize_block16(A, layout="blocked")
        qw, sw, tw = spg.quantize_block16(W, layout="blocked")
        out = spg.gemm_scaled(qa, sa, qw, sw, wl.epilogue, residual=R, fmt="nvfp4", tscale_a=ta, tscale_w=tw,
                              scale_layout="blocked")
    torch.cuda.synchronize()
    gpu = host_u16(out)
    del A, W, R, qa, qw, out
    torch.cuda.empty_cache()

    batches = list(range(wl.batch)) if wl.batch > 1 else [None]
    for b in batches:
        Ab = A16[b] if b is not None else A16
        Wb = W16[b] if b is not None else W16
        g = gpu[b] if b is not None else gpu
        # every 256-row tile row and every tile column (SwiGLU: 128 outputs)
        # twice, one index in each half: with the persistent walk, the K-split
        # tail and both halves of half-height tail tiles, every tile is hit
        rows = sample_every_tile(wl.M, rng, 256)
        cols = sample_every_tile(wl.n_out, rng, 128 if wl.epilogue == "swiglu" else 256)
        tiles_m = -(-wl.M // 256)
        tiles_n = -(-wl.n_out // (128 if wl.epilogue == "swiglu" else 256))
        assert len(np.unique(rows // 256)) == tiles_m
        assert len(np.unique(cols // (128 if wl.epilogue == "swiglu" else 256))) == tiles_n
        wrows = np.concatenate([cols, cols + wl.N // 2]) if wl.epilogue == "swiglu" else cols
        Rb = np.broadcast_to(R16, (wl.M, wl.n_out)) if wl.bias else R16
        Rs = np.ascontiguousarray(Rb[np.ix_(rows, cols)]) if R16 is not None else None
        if wl.fmt == "e4m3_row":
            qa_o, sa_o = oracle.quantize_rowwise(np.ascontiguousarray(Ab[rows]))
            qw_o, sw_o = oracle.quantize_rowwise(np.ascontiguousarray(Wb[wrows]))
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        elif wl.fmt == "e4m3_tensor":
            sa_o = oracle.amax(Ab) / np.float32(448.0)
            sw_o = oracle.amax(Wb) / np.float32(448.0)
            qa_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(Ab[rows]), sa_o)
            qw_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(Wb[wrows]), sw_o)
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        else:
            ta_o = oracle.nvfp4_tensor_scale(Ab)
            tw_o = oracle.nvfp4_tensor_scale(Wb)
            qa_o, bsa_o = oracle.quantize_block16_rows(np.ascontiguousarray(Ab[rows]), ta_o)
            qw_o, bsw_o = oracle.quantize_block16_rows(np.ascontiguousarray(Wb[wrows]), tw_o)
            D, Da = oracle.gemm_nvfp4_sums(qa_o, bsa_o, qw_o, bsw_o)
            sa_o, sw_o = ta_o, tw_o
        y, S, _ = oracle.epilogue(wl.epilogue, D, Da, sa_o, sw_o, Rs)
        check_close(np.ascontiguousarray(g[np.ix_(rows, cols)]), y, S, f"{name} batch {b}")


# ---------------------------------------------------------------------------
# tail split: 272 tiles on 256 compute units; the last 16 tiles (tile rows
# 8..15, tile columns 15 and 16 in the raster order) run split along K in a
# second launch.  Outputs are sampled in both parts.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,K", [("nvfp4", 4096), ("e4m3_row", 16384)])
def test_gemm_tail_split_sampled(spg, fmt, K):
    M, N = 4096, 4352
    plan = spg.gemm_plan(M, N, K, fmt, "store")
    assert plan["tail_tiles"] == 16 and plan["tail_split"] > 1
    rng = np.random.default_rng(123)
    A16 = bf16_normal((M, K), 1.0, 70)
    W16 = bf16_normal((N, K), 0.02, 71)
    A, W = dev(A16), dev(W16)
    if fmt == "nvfp4":
        qa, sa, ta = spg.quantize_block16(A)
        qw, sw, tw = spg.quantize_block16(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, "store", fmt="nvfp4", tscale_a=ta, tscale_w=tw)
    else:
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, "store")
    torch.cuda.synchronize()
    gpu = host_u16(out)
    del A, W, qa, qw, out
    torch.cuda.empty_cache()
    rows = np.unique(np.concatenate([sample(M, 24, rng), rng.choice(np.arange(2048, M), 16, replace=False)]))
    cols = np.unique(np.concatenate([sample(N, 24, rng), rng.choice(np.arange(3840, N), 16, replace=False), [3840, N - 1]]))
    if fmt == "nvfp4":
        ta_o, tw_o = oracle.nvfp4_tensor_scale(A16), oracle.nvfp4_tensor_scale(W16)
        qa_o, bsa_o = oracle.quantize_block16_rows(np.ascontiguousarray(A16[rows]), ta_o)
        qw_o, bsw_o = oracle.quantize_block16_rows(np.ascontiguousarray(W16[cols]), tw_o)
        D, Da = oracle.gemm_nvfp4_sums(qa_o, bsa_o, qw_o, bsw_o)
        y, S, _ = oracle.epilogue("store", D, Da, ta_o, tw_o, None)
    else:
        qa_o, sa_o = oracle.quantize_rowwise(np.ascontiguousarray(A16[rows]))
        qw_o, sw_o = oracle.quantize_rowwise(np.ascontiguousarray(W16[cols]))
        D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        y, S, _ = oracle.epilogue("store", D, Da, sa_o, sw_o, None)
    check_close(np.ascontiguousarray(gpu[np.ix_(rows, cols)]), y, S, f"tail split {fmt} K={K}")


# ---------------------------------------------------------------------------
# half-height tail: 272 (or 544) tiles on 256 compute units; the last round's
# tiles run as 128-row halves in a second launch.  Every output column of the
# tail's tile columns is checked on sampled rows of both halves, with ragged
# M (a last tile row whose lower half is partly or wholly empty), ragged N, a
# K tail inside a stage, SwiGLU pairing and per-tensor batches.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,epi,fmt,B", [
    (4096, 4352, 2048, "store", "e4m3_row", 1),
    (4000, 4312, 2064, "add", "e4m3_row", 1),
    (3900, 8704, 1024, "swiglu", "e4m3_row", 1),
    (2048, 4352, 2048, "store", "e4m3_tensor", 2),
    (4000, 4312, 2064, "bias", "e4m3_row", 1),
    (4000, 4312, 2064, "bias8", "e4m3_row", 1),
], ids=["store", "add_ragged", "swiglu_ragged", "tensor_batch2", "bias_ragged", "e4m3_bias_ragged"])
def test_gemm_half_tail(spg, M, N, K, epi, fmt, B):
    bias8 = epi == "bias8"      # ADD with an E4M3 bias row and its scale
    bias = epi == "bias"        # ADD with one bf16 row broadcast to every token row
    epi = "add" if (bias or bias8) else epi
    plan = spg.gemm_plan(M, N, K, fmt, epi, batch=B)
    assert plan["tail_bm"] == 128 and plan["tail_tiles"] in (16, 32) and plan["tail_split"] == 1
    rng = np.random.default_rng(M + N + K)
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, 80)
    W16 = bf16_normal((N, K), 0.02, 81)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, 82) if epi == "add" else None
    res = dev(R16) if R16 is not None else None
    bscale, bvals = None, None
    if bias:
        row = bf16_normal((n_out,), 1.0, 83)
        R16, res = np.broadcast_to(row, (M, n_out)), dev(row)
    if bias8:
        res, bscale, bvals = e4m3_bias(spg, bf16_normal((n_out,), 1.0, 84))
        R16 = None
    A, W = dev(A16), dev(W16)
    if fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res, bias_scale=bscale)
    else:
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, epi, fmt="e4m3_tensor")
    torch.cuda.synchronize()
    gpu = host_u16(out)
    del A, W, qa, qw, out
    torch.cuda.empty_cache()
    # tail tile columns: the last tiles in the raster order sit in the last
    # group of eight tile rows, at the highest tile columns
    tile_n = 128 if epi == "swiglu" else 256
    first_tail_col = ((n_out + tile_n - 1) // tile_n - (2 if plan["tail_tiles"] == 16 else 4)) * tile_n
    cols = np.unique(np.concatenate([sample(n_out, 16, rng), np.arange(first_tail_col, n_out)]))
    wrows = np.concatenate([cols, cols + N // 2]) if epi == "swiglu" else cols
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        g = gpu[b] if B > 1 else gpu
        last = ((M - 1) // 256) * 256       # first row of the last tile row
        rows = np.unique(np.concatenate([sample(M, 24, rng), rng.choice(np.arange(M // 2, M), 24, replace=False),
                                         [M // 2, M // 2 + 127, M // 2 + 128, last, min(last + 127, M - 1),
                                          min(last + 128, M - 1), M - 1]]))
        Rs = np.ascontiguousarray(R16[np.ix_(rows, cols)]) if R16 is not None else None
        if fmt == "e4m3_row":
            qa_o, sa_o = oracle.quantize_rowwise(np.ascontiguousarray(Ab[rows]))
            qw_o, sw_o = oracle.quantize_rowwise(np.ascontiguousarray(W16[wrows]))
        else:
            sa_o = oracle.amax(Ab) / np.float32(448.0)
            sw_o = oracle.amax(W16) / np.float32(448.0)
            qa_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(Ab[rows]), sa_o)
            qw_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(W16[wrows]), sw_o)
        D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        y, S, _ = oracle.epilogue(epi, D, Da, sa_o, sw_o, Rs, None if bvals is None else bvals[cols])
        check_close(np.ascontiguousarray(g[np.ix_(rows, cols)]), y, S, f"half tail {M}x{N}x{K} {epi} {fmt} batch {b}")


# ---------------------------------------------------------------------------
# the half-height kernel over a grid of 128-row tiles for a whole product,
# several rounds of workgroups and raster groups of eight tile rows (the last
# one partial), ragged M, N and K: two rows of every 128-row tile row (its
# first and its last) and two columns of every tile column are checked, plus
# random ones.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,epi,fmt,B", [
    (4096, 4352, 1024, "store", "e4m3_row", 1),
    (4000, 4312, 1040, "add", "e4m3_row", 1),
    (2048, 4352, 1024, "store", "e4m3_tensor", 2),
    (700, 8704, 1040, "swiglu", "e4m3_row", 1),
    (1100, 7168, 512, "bias8", "e4m3_row", 1),
], ids=["store_3_rounds", "add_ragged", "tensor_batch2", "swiglu_ragged", "e4m3_bias_ragged"])
def test_gemm_half_grid_sampled(spg, M, N, K, epi, fmt, B):
    bias8 = epi == "bias8"
    epi = "add" if bias8 else epi
    plan = spg.gemm_plan(M, N, K, fmt, epi, batch=B)
    tile_n = 128 if epi == "swiglu" else 256
    n_out = N // 2 if epi == "swiglu" else N
    assert plan["kernel"] == 2 and plan["workgroups"] == B * -(-M // 128) * -(-n_out // tile_n)
    rng = np.random.default_rng(M + N + K + B)
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, 60)
    W16 = bf16_normal((N, K), 0.02, 61)
    R16 = bf16_normal((M, n_out), 1.0, 62) if epi == "add" and not bias8 else None
    res, bscale, bvals = (dev(R16) if R16 is not None else None), None, None
    if bias8:
        res, bscale, bvals = e4m3_bias(spg, bf16_normal((n_out,), 1.0, 63))
    A, W = dev(A16), dev(W16)
    if fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res, bias_scale=bscale)
    else:
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, epi, fmt="e4m3_tensor")
    torch.cuda.synchronize()
    gpu = host_u16(out)
    del A, W, qa, qw, out
    torch.cuda.empty_cache()
    firsts = np.arange(0, M, 128)
    rows = np.unique(np.concatenate([firsts, np.minimum(firsts + 127, M - 1), sample(M, 16, rng)]))
    cfirst = np.arange(0, n_out, tile_n)
    cols = np.unique(np.concatenate([cfirst, np.minimum(cfirst + tile_n - 1, n_out - 1), sample(n_out, 16, rng)]))
    wrows = np.concatenate([cols, cols + N // 2]) if epi == "swiglu" else cols
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        Rs = np.ascontiguousarray(R16[np.ix_(rows, cols)]) if R16 is not None else None
        if fmt == "e4m3_row":
            qa_o, sa_o = oracle.quantize_rowwise(np.ascontiguousarray(Ab[rows]))
            qw_o, sw_o = oracle.quantize_rowwise(np.ascontiguousarray(W16[wrows]))
        else:
            sa_o = oracle.amax(Ab) / np.float32(448.0)
            sw_o = oracle.amax(W16) / np.float32(448.0)
            qa_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(Ab[rows]), sa_o)
            qw_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(W16[wrows]), sw_o)
        D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        y, S, _ = oracle.epilogue(epi, D, Da, sa_o, sw_o, Rs, None if bvals is None else bvals[cols])
        g = gpu[b] if B > 1 else gpu
        check_close(np.ascontiguousarray(g[np.ix_(rows, cols)]), y, S, f"half grid {M}x{N}x{K} {epi} {fmt} batch {b}")


# ---------------------------------------------------------------------------
# 65 - 128 tokens: unsplit FP8 products run as one row of 128-row half tiles
# (the lower half of a 256-row tile would be empty).  Whole outputs: ragged
# M, N and K, a single K stage, a K tail inside the first stage, SwiGLU
# pairing, both scale forms, and more tile columns than compute units (257:
# a second round of workgroups).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,epi,fmt", [
    (65, 700, 1040, "store", "e4m3_row"),
    (100, 600, 512, "swiglu", "e4m3_row"),
    (128, 1000, 384, "add", "e4m3_tensor"),
    (97, 520, 128, "add", "e4m3_row"),
    (128, 300, 16, "swiglu", "e4m3_tensor"),
    (128, 65792, 256, "store", "e4m3_row"),
], ids=["ragged_store", "swiglu", "tensor_add", "one_stage", "k16", "257_tiles"])
def test_gemm_half_route_up_to_128_tokens(spg, M, N, K, epi, fmt):
    plan = spg.gemm_plan(M, N, K, fmt, epi)
    assert plan["kernel"] == 2 and plan["bm"] == 128 and plan["workgroups"] == plan["tiles"]
    A16 = bf16_normal((M, K), 1.0, 70 + M)
    W16 = bf16_normal((N, K), 0.02, 71 + N)
    R16 = bf16_normal((M, N), 1.0, 72) if epi == "add" else None
    gpu = run_fp8(spg, A16, W16, epi, fmt, R16)
    ref = oracle_fp8(A16, W16, epi, fmt, R16)
    check_close(gpu, ref["y"], ref["S"], f"half route {M}x{N}x{K} {epi} {fmt}")


# ---------------------------------------------------------------------------
# SwiGLU with gate values far below zero (unit-variance weights, long K):
# where 1 + exp(-g) leaves the range whose reciprocal is a normal float, the
# epilogue switches to the limit form g u exp(g); outputs down to bf16's
# subnormals must still match.  Every route: 128-row tiles, 256-row tiles,
# the split-K reduction, the decode-width kernel, NVFP4.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,M,N,K,kernel,split", [
    ("e4m3_tensor", 300, 1024, 1536, 2, False),
    ("e4m3_tensor", 512, 16896, 512, 0, False),
    ("e4m3_tensor", 64, 1024, 8192, 0, True),
    ("e4m3_tensor", 16, 1024, 4096, 3, False),
    ("nvfp4", 512, 2048, 1536, 1, False),
    ("nvfp4", 256, 1024, 4096, 1, True),
], ids=["half_tiles", "full_tiles", "split_k", "decode_width", "nvfp4", "nvfp4_split_k"])
def test_swiglu_far_negative_gates(spg, fmt, M, N, K, kernel, split):
    plan = spg.gemm_plan(M, N, K, fmt, "swiglu")
    assert plan["kernel"] == kernel and (plan["split_k"] > 1) == split
    A16 = bf16_normal((M, K), 1.0, 30 + M)
    W16 = bf16_normal((N, K), 1.0, 31 + K)
    if fmt == "nvfp4":
        gpu = run_nvfp4(spg, A16, W16, "swiglu")
        qa, bsa, ta = oracle.quantize_block16(A16)
        qw, bsw, tw = oracle.quantize_block16(W16)
        D, Da = oracle.gemm_nvfp4_sums(qa, bsa, qw, bsw)
        sc = float(ta) * float(tw)
        y, S, _ = oracle.epilogue("swiglu", D, Da, ta, tw, None)
    else:
        gpu = run_fp8(spg, A16, W16, "swiglu", fmt)
        qa, sa = oracle.quantize_tensor(A16)
        qw, sw = oracle.quantize_tensor(W16)
        D, Da = oracle.gemm_e4m3_sums(qa, qw)
        sc = float(sa[0]) * float(sw[0])
        y, S, _ = oracle.epilogue("swiglu", D, Da, sa[0], sw[0], None)
    gate = D[:, : N // 2] * sc
    assert np.count_nonzero(gate < -88.0) > 0 and np.count_nonzero((gate < -80.0) & (np.abs(y) > 2.0 ** -126)) > 0
    check_close(gpu, y, S, f"far negative gates {fmt} {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# bf16 bias: the ADD epilogue with one residual row (row stride 0) added to
# every token row - unsplit tiles, several tiles per persistent workgroup,
# split-K with its reduction (many and few tokens), both FP8 scale forms and
# NVFP4, and a batch sharing the bias.
# ---------------------------------------------------------------------------

BIAS = [((128, 256, 512), "e4m3_row", 1), ((300, 258, 1040), "e4m3_tensor", 1), ((17, 34, 48), "e4m3_row", 1),
        ((2304, 7936, 256), "e4m3_row", 1), ((520, 1030, 2064), "e4m3_row", 1), ((16, 5120, 17408), "e4m3_row", 1),
        ((96, 300, 512), "e4m3_tensor", 3), ((257, 300, 512), "nvfp4", 1), ((64, 64, 256), "nvfp4", 1),
        ((20, 1000, 1040), "e4m3_row", 1), ((8, 520, 512), "nvfp4", 1), ((6, 520, 256), "e4m3_tensor", 2)]


@pytest.mark.parametrize("shape,fmt,B", BIAS, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_gemm_bias_row(spg, shape, fmt, B):
    M, N, K = shape
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, 90 + M)
    W16 = bf16_normal((N, K), 0.02, 91 + N)
    row = bf16_normal((N,), 1.0, 92 + K)
    A, W, bias = dev(A16), dev(W16), dev(row)
    if fmt == "nvfp4":
        qa, bsa, ta = spg.quantize_block16(A)
        qw, bsw, tw = spg.quantize_block16(W)
        out = spg.gemm_scaled(qa, bsa, qw, bsw, "add", residual=bias, fmt="nvfp4", tscale_a=ta, tscale_w=tw)
    elif fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, "add", residual=bias)
    else:
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, "add", residual=bias, fmt="e4m3_tensor")
    gpu = host_u16(out)
    R16 = np.broadcast_to(row, (M, N))
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        if fmt == "nvfp4":
            ref = oracle_nvfp4(Ab, W16, "add", R16)
        elif fmt == "e4m3_row":
            ref = oracle_fp8(Ab, W16, "add", "e4m3_row", R16)
        else:
            # the batch's per-tensor scales: each entry's own amax
            qa_o, sa_o = oracle.quantize_tensor(Ab)
            qw_o, sw_o = oracle.quantize_tensor(W16)
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
            y, S, o = oracle.epilogue("add", D, Da, sa_o[0], sw_o[0], R16)
            ref = dict(y=y, S=S, out=o)
        check_close(gpu[b] if B > 1 else gpu, ref["y"], ref["S"], f"bias {shape} {fmt} batch {b}")


def test_gemm_bias_row_with_zero_weights_is_the_bias(spg):
    # every product is zero: each output row is the bias, bit for bit, also
    # through split-K (16 tokens over a long K) and its reduction
    for M, N, K in [(300, 260, 256), (16, 520, 8192)]:
        A16 = bf16_normal((M, K), 1.0, 7)
        row = bf16_normal((N,), 1.0, 8)
        gpu = run_fp8(spg, A16, np.zeros((N, K), np.uint16), "add", "e4m3_row", row)
        assert np.array_equal(gpu, np.tile(row, (M, 1))), (M, N, K)


# ---------------------------------------------------------------------------
# FP8 bias: the bias row stored as E4M3 codes with one fp32 scale (made by
# the row quantizer from a bf16 row), dequantized in the epilogue after the
# operand scales (AstrAI commit log, the commit fusing the bias).  The same
# routes as the bf16 bias row: 256- and 128-row tiles, persistent
# workgroups, split-K and its reduction, per-tensor batches, NVFP4.
# ---------------------------------------------------------------------------

def e4m3_bias(spg, row16):
    """(codes uint8 [N], scale fp32 [1]) on the device, and the oracle's
    dequantized values for the same row (the codes checked equal).  The
    device quantizer takes rows of a multiple of 16 values: the row is
    padded with zeros, which leave its amax, scale and codes unchanged."""
    n = row16.shape[0]
    padded = np.zeros((1, (n + 15) // 16 * 16), np.uint16)
    padded[0, :n] = row16
    q, s = spg.quantize_rowwise(dev(padded))
    q_o, s_o = oracle.quantize_rowwise(row16[None, :])
    assert np.array_equal(q.cpu().numpy()[:, :n], q_o) and s.cpu().numpy()[0] == s_o[0]
    return q[0, :n].contiguous(), s, oracle.bias_e4m3(q_o[0], s_o[0])


@pytest.mark.parametrize("shape,fmt,B", BIAS, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_gemm_e4m3_bias_row(spg, shape, fmt, B):
    M, N, K = shape
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, 190 + M)
    W16 = bf16_normal((N, K), 0.02, 191 + N)
    row = bf16_normal((N,), 0.5, 192 + K)
    codes, bscale, bvals = e4m3_bias(spg, row)
    A, W = dev(A16), dev(W16)
    if fmt == "nvfp4":
        qa, bsa, ta = spg.quantize_block16(A)
        qw, bsw, tw = spg.quantize_block16(W)
        out = spg.gemm_scaled(qa, bsa, qw, bsw, "add", residual=codes, fmt="nvfp4", tscale_a=ta, tscale_w=tw,
                              bias_scale=bscale)
    elif fmt == "e4m3_row":
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, "add", residual=codes, bias_scale=bscale)
    else:
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        out = spg.gemm_scaled(qa, sa, qw, sw, "add", residual=codes, fmt="e4m3_tensor", bias_scale=bscale)
    gpu = host_u16(out)
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        if fmt == "nvfp4":
            qa_o, bsa_o, ta_o = oracle.quantize_block16(Ab)
            qw_o, bsw_o, tw_o = oracle.quantize_block16(W16)
            D, Da = oracle.gemm_nvfp4_sums(qa_o, bsa_o, qw_o, bsw_o)
            y, S, _ = oracle.epilogue("add", D, Da, ta_o, tw_o, bias=bvals)
        else:
            if fmt == "e4m3_row":
                qa_o, sa_o = oracle.quantize_rowwise(Ab)
                qw_o, sw_o = oracle.quantize_rowwise(W16)
            else:
                qa_o, sa_o = oracle.quantize_tensor(Ab)
                qw_o, sw_o = oracle.quantize_tensor(W16)
                sa_o, sw_o = sa_o[0], sw_o[0]
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
            y, S, _ = oracle.epilogue("add", D, Da, sa_o, sw_o, bias=bvals)
        check_close(gpu[b] if B > 1 else gpu, y, S, f"e4m3 bias {shape} {fmt} batch {b}")


def test_gemm_e4m3_bias_with_zero_weights_is_the_bias(spg):
    # zero weights: every row is the dequantized bias.  With a power-of-two
    # bias scale dec(code) * scale is exact in fp32, so the output is the
    # oracle's one rounding bit for bit - also through a 128-row tile
    # product, the persistent kernel and split-K with its reduction
    rng = np.random.default_rng(5)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for M, N, K in [(300, 260, 256), (2304, 520, 128), (16, 520, 8192)]:
        A16 = bf16_normal((M, K), 1.0, 9)
        codes = rng.choice(finite, size=(N,)).astype(np.uint8)
        scale = np.float32(2.0 ** -7)
        A = dev(A16)
        qa, sa = spg.quantize_rowwise(A)
        qw = torch.zeros((N, K), dtype=torch.uint8, device="cuda")
        sw = torch.ones((N,), dtype=torch.float32, device="cuda")
        out = spg.gemm_scaled(qa, sa, qw, sw, "add", residual=torch.from_numpy(codes).cuda(),
                              bias_scale=torch.tensor([scale], device="cuda"))
        gpu = host_u16(out)
        # the oracle's epilogue on zero sums (a -0 bias gives +0 after the add)
        _, _, want = oracle.epilogue("add", np.zeros((1, N)), np.zeros((1, N)), 1.0, 1.0,
                                     bias=oracle.bias_e4m3(codes, scale))
        assert np.array_equal(gpu, np.tile(want, (M, 1))), (M, N, K)


# ---------------------------------------------------------------------------
# Split-N outputs (the fused input projections of ninfer PR #167's call-site
# list): one GEMM, each column range into its own tensor.  Every segment must
# equal the same columns of the unsplit output bit for bit (the same kernels
# run; only the store addresses differ) and match the oracle - through 128-row
# tiles, a K split with its reduction, few tokens, SwiGLU, a residual with a
# ragged last segment, per-tensor batches and NVFP4.
# ---------------------------------------------------------------------------

SPLITS = [((300, 640, 512), "e4m3_row", "store", (256, 256, 128), 1),
          ((1024, 768, 2048), "e4m3_row", "store", (384, 384), 1),
          ((16, 5120, 4096), "e4m3_row", "store", (4096, 512, 512), 1),
          ((300, 1280, 512), "e4m3_row", "swiglu", (384, 256), 1),
          ((520, 1030, 1024), "e4m3_row", "add", (512, 448, 70), 1),
          ((96, 300, 512), "e4m3_tensor", "store", (256, 44), 2),
          ((257, 640, 512), "nvfp4", "store", (64, 512, 64), 1),
          ((20, 1280, 1024), "e4m3_row", "swiglu", (384, 256), 1),
          ((8, 640, 512), "nvfp4", "store", (64, 512, 64), 1),
          ((4, 1100, 256), "e4m3_row", "add", (512, 448, 140), 1),
          ((260, 700, 512), "e4m3_tensor", "store", (256, 384, 60), 2)]


@pytest.mark.parametrize("shape,fmt,epi,widths,B", SPLITS,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_gemm_out_split(spg, shape, fmt, epi, widths, B):
    M, N, K = shape
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, 300 + M)
    W16 = bf16_normal((N, K), 0.02, 301 + N)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, 302) if epi == "add" else None
    A, W = dev(A16), dev(W16)
    res = dev(R16) if R16 is not None else None
    if fmt == "nvfp4":
        qa, bsa, ta = spg.quantize_block16(A)
        qw, bsw, tw = spg.quantize_block16(W)
        run = lambda **kw: spg.gemm_scaled(qa, bsa, qw, bsw, epi, residual=res, fmt="nvfp4", tscale_a=ta,
                                           tscale_w=tw, **kw)
    else:
        q = spg.quantize_rowwise if fmt == "e4m3_row" else spg.quantize_tensor
        qa, sa = q(A)
        qw, sw = q(W)
        run = lambda **kw: spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res, fmt=fmt, **kw)
    whole = run()
    segs = run(out_split=list(widths))
    torch.cuda.synchronize()
    assert [t.shape[-1] for t in segs] == list(widths)
    assert torch.equal(torch.cat(segs, dim=-1).view(torch.int16), whole.view(torch.int16))
    gpu = host_u16(torch.cat(segs, dim=-1))
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        ref = oracle_nvfp4(Ab, W16, epi, R16) if fmt == "nvfp4" else oracle_fp8(Ab, W16, epi, fmt, R16)
        check_close(gpu[b] if B > 1 else gpu, ref["y"], ref["S"], f"split {shape} {fmt} {epi} batch {b}")


def test_gemm_out_split_into_strided_views(spg):
    # segments as column windows of wider buffers (row stride > width): the
    # windows get the output, the rest of each buffer is left as it was
    M, N, K = 520, 768, 1024
    A16 = bf16_normal((M, K), 1.0, 310)
    W16 = bf16_normal((N, K), 0.02, 311)
    qa, sa = spg.quantize_rowwise(dev(A16))
    qw, sw = spg.quantize_rowwise(dev(W16))
    whole = spg.gemm_scaled(qa, sa, qw, sw, "store")
    bufs = [torch.full((M, 512), 7.0, dtype=torch.bfloat16, device="cuda"),
            torch.full((M, 704), -3.0, dtype=torch.bfloat16, device="cuda")]
    views = [bufs[0][:, 64:448], bufs[1][:, 320:704]]
    out = spg.gemm_scaled(qa, sa, qw, sw, "store", out_split=views)
    torch.cuda.synchronize()
    assert out[0].data_ptr() == views[0].data_ptr()
    assert torch.equal(bufs[0][:, 64:448].view(torch.int16), whole[:, :384].view(torch.int16))
    assert torch.equal(bufs[1][:, 320:704].view(torch.int16), whole[:, 384:].view(torch.int16))
    assert torch.all(bufs[0][:, :64] == 7.0) and torch.all(bufs[0][:, 448:] == 7.0)
    assert torch.all(bufs[1][:, :320] == -3.0)


@pytest.mark.parametrize("name", ["fp8_row_attn_in_t4096", "fp8_row_gdn_in_t4096"])
def test_workload_out_split_full_size(spg, name):
    # the two projection workloads at full size: bitwise against the unsplit
    # output, and the oracle on rows and columns that reach every tile
    wl = WORKLOADS[name]
    rng = np.random.default_rng(wl.seed)
    A16, W16, _ = wl.inputs()
    qa, sa = spg.quantize_rowwise(dev(A16))
    qw, sw = spg.quantize_rowwise(dev(W16))
    whole = spg.gemm_scaled(qa, sa, qw, sw, wl.epilogue)
    segs = spg.gemm_scaled(qa, sa, qw, sw, wl.epilogue, out_split=list(wl.split))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(segs, dim=-1).view(torch.int16), whole.view(torch.int16))
    del whole
    rows = sample_every_tile(wl.M, rng, 256)
    cols = sample_every_tile(wl.n_out, rng, 256)
    bounds = np.cumsum((0,) + wl.split)
    # both sides of every segment boundary
    cols = np.unique(np.concatenate([cols, bounds[1:-1], bounds[1:-1] - 1]))
    gpu = np.concatenate([host_u16(t[torch.from_numpy(rows).cuda()]) for t in segs], axis=1)[:, cols]
    ref = oracle.linear_e4m3_rowwise(np.ascontiguousarray(A16[rows]), np.ascontiguousarray(W16[cols]), "store")
    check_close(gpu, ref["y"], ref["S"], f"{name} sampled")


# ---------------------------------------------------------------------------
# K-major operands (the backward products' layouts: dX = dY W reads W as
# [K, N], dW = dY^T X reads both operands K-major).  The call must equal the
# NT product of the explicitly transposed codes bit for bit (it transposes
# into the workspace and runs the same kernels) and match the oracle:
# ragged shapes with padded row strides, few tokens through a K split (its
# partials sit behind the transposed copies in the workspace), batches.
# ---------------------------------------------------------------------------

def kmajor(codes: torch.Tensor, ld: int) -> torch.Tensor:
    """[.., R, K] codes stored K-major as [.., K, R] with row stride ld >= R."""
    t = codes.transpose(-1, -2)
    buf = torch.zeros(t.shape[:-1] + (ld,), dtype=torch.uint8, device=codes.device)
    buf[..., : t.shape[-1]] = t
    return buf[..., : t.shape[-1]]


KMAJOR = [((300, 520, 1040), "e4m3_tensor", "store", (False, True), 1),
          ((300, 520, 1040), "e4m3_tensor", "add", (True, True), 1),
          ((257, 300, 512), "e4m3_row", "swiglu", (True, False), 1),
          ((16, 4096, 2048), "e4m3_row", "store", (False, True), 1),
          ((96, 200, 256), "e4m3_tensor", "store", (True, True), 2),
          ((1024, 2048, 4096), "e4m3_tensor", "store", (True, True), 1),
          ((260, 520, 512), "e4m3_tensor", "add", (True, True), 2)]


@pytest.mark.parametrize("shape,fmt,epi,km,B", KMAJOR,
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_gemm_kmajor_operands(spg, shape, fmt, epi, km, B):
    M, N, K = shape
    a_km, w_km = km
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, 400 + M)
    W16 = bf16_normal((N, K), 0.02 if fmt == "e4m3_row" else 1.0, 401 + N)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, 402) if epi == "add" else None
    res = dev(R16) if R16 is not None else None
    q = spg.quantize_rowwise if fmt == "e4m3_row" else spg.quantize_tensor
    qa, sa = q(dev(A16))
    qw, sw = q(dev(W16))
    nt = spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res, fmt=fmt)
    ka = kmajor(qa, (M + 31) // 32 * 32) if a_km else qa
    kw = kmajor(qw, (N + 15) // 16 * 16 + 16) if w_km else qw
    got = spg.gemm_scaled(ka, sa, kw, sw, epi, residual=res, fmt=fmt, a_kmajor=a_km, w_kmajor=w_km)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), nt.view(torch.int16))
    gpu = host_u16(got)
    rng = np.random.default_rng(M + N)
    big = M * N > 1 << 21
    rows = sample_every_tile(M, rng, 256) if big else np.arange(M)
    cols = sample_every_tile(n_out, rng, 128) if big else np.arange(n_out)
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        g = gpu[b] if B > 1 else gpu
        if big:
            # per-tensor scales over the whole matrices, codes of the sampled rows
            sa_o = oracle.amax(Ab) / np.float32(448.0)
            sw_o = oracle.amax(W16) / np.float32(448.0)
            qa_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(Ab[rows]), sa_o)
            qw_o = oracle.quantize_rows_with_scale(np.ascontiguousarray(W16[cols]), sw_o)
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
            y, S, _ = oracle.epilogue(epi, D, Da, sa_o, sw_o)
            check_close(np.ascontiguousarray(g[np.ix_(rows, cols)]), y, S, f"kmajor {shape} sampled")
        else:
            if fmt == "e4m3_tensor" and B > 1:
                qa_o, sa_o = oracle.quantize_tensor(Ab)
                qw_o, sw_o = oracle.quantize_tensor(W16)
                D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
                y, S, _ = oracle.epilogue(epi, D, Da, sa_o[0], sw_o[0], R16)
                ref = dict(y=y, S=S)
            else:
                ref = oracle_fp8(Ab, W16, epi, fmt, R16)
            check_close(g, ref["y"], ref["S"], f"kmajor {shape} {fmt} {epi} {km} batch {b}")


# ---------------------------------------------------------------------------
# few tokens (M <= 64).  At most 32 tokens with at least 32 blocks of 16
# output columns: the decode-width kernel (one workgroup per 16 columns, K
# split over its waves) - one and two token blocks (M <= 16, 17..32), ragged
# column blocks (SwiGLU halves that are not a multiple of 4 columns), K
# tails inside a 128-byte chunk and K below one chunk (waves without work).
# Otherwise the tiled few-token route: one partly filled tile row, K split
# over many slices (instantiations for at most 32 and at most 64 tokens).
# Per-tensor batches with a broadcast or a per-batch weight, and the two
# prefill linears at 16 tokens.
# ---------------------------------------------------------------------------

NARROW = [((1, 64, 256), "store", "e4m3_row"), ((5, 200, 1040), "add", "e4m3_row"),
          ((16, 2060, 528), "swiglu", "e4m3_row"), ((31, 130, 4112), "store", "e4m3_tensor"),
          ((32, 520, 2048), "add", "e4m3_tensor"), ((7, 34, 48), "swiglu", "e4m3_tensor"),
          ((16, 5120, 17408), "add", "e4m3_row"), ((16, 34816, 5120), "swiglu", "e4m3_row"),
          ((33, 300, 1040), "store", "e4m3_row"), ((48, 2060, 528), "swiglu", "e4m3_tensor"),
          ((64, 5120, 4096), "add", "e4m3_row"),
          ((1, 1000, 1040), "store", "e4m3_row"), ((17, 600, 4112), "add", "e4m3_row"),
          ((5, 1034, 528), "swiglu", "e4m3_tensor"), ((32, 1024, 128), "swiglu", "e4m3_row"),
          ((24, 700, 80), "add", "e4m3_tensor"), ((2, 4096, 16), "store", "e4m3_row")]


@pytest.mark.parametrize("shape,epi,fmt", NARROW, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_gemm_narrow(spg, shape, epi, fmt):
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, 4 * M + K)
    W16 = bf16_normal((N, K), 0.02, 6 * N + K)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, M + N + 2) if epi == "add" else None
    gpu = run_fp8(spg, A16, W16, epi, fmt, R16)
    ref = oracle_fp8(A16, W16, epi, fmt, R16)
    assert gpu.shape == ref["out"].shape
    check_close(gpu, ref["y"], ref["S"], f"narrow {shape} {epi} {fmt}")


@pytest.mark.parametrize("N", [300, 600], ids=["tiled", "decode_width"])
def test_gemm_narrow_batched_broadcast_and_deterministic(spg, N):
    B, M, K = 3, 9, 1536
    A16 = bf16_normal((B, M, K), 1.0, 91)
    W16 = bf16_normal((N, K), 0.02, 92)
    qa, sa = spg.quantize_tensor(dev(A16))
    qw, sw = spg.quantize_tensor(dev(W16))
    out1 = host_u16(spg.gemm_scaled(qa, sa, qw, sw, "store", fmt="e4m3_tensor"))
    out2 = host_u16(spg.gemm_scaled(qa, sa, qw, sw, "store", fmt="e4m3_tensor"))
    assert np.array_equal(out1, out2)
    qwo, swo = oracle.quantize_tensor(W16)
    for b in range(B):
        qao, sao = oracle.quantize_tensor(A16[b])
        D, Da = oracle.gemm_e4m3_sums(qao, qwo)
        y, S, _ = oracle.epilogue("store", D, Da, sao[0], swo[0])
        check_close(out1[b], y, S, f"narrow batch {b}")


@pytest.mark.parametrize("M,K", [(8, 512), (32, 512), (100, 512), (300, 512), (300, 2048)],
                         ids=["decode_width", "decode_width_two_blocks", "half_tiles", "half_tiles_3_rows", "split_k"])
def test_gemm_row_scaled_batches_with_residual(spg, M, K):
    # row scales per batch entry (A and W rows of every entry have their own),
    # per-entry weights, a batched residual
    B, N = 2, 600
    A16 = bf16_normal((B, M, K), 1.0, 95 + M)
    W16 = bf16_normal((B, N, K), 0.02, 96)
    R16 = bf16_normal((B, M, N), 1.0, 97)
    qa = torch.stack([spg.quantize_rowwise(dev(A16[b]))[0] for b in range(B)])
    sa = torch.stack([spg.quantize_rowwise(dev(A16[b]))[1] for b in range(B)])
    qw = torch.stack([spg.quantize_rowwise(dev(W16[b]))[0] for b in range(B)])
    sw = torch.stack([spg.quantize_rowwise(dev(W16[b]))[1] for b in range(B)])
    assert spg.gemm_plan(M, N, K, "e4m3_row", "add", batch=B)["kernel"] == (3 if M <= 32 else 0 if K > 1024 else 2)
    out = host_u16(spg.gemm_scaled(qa, sa, qw, sw, "add", residual=dev(R16)))
    for b in range(B):
        ref = oracle_fp8(A16[b], W16[b], "add", "e4m3_row", R16[b])
        check_close(out[b], ref["y"], ref["S"], f"row-scaled batch {b} M={M}")


def test_gemm_narrow_batched_per_batch_weights(spg):
    # per-tensor products with a weight of their own per batch entry
    B, M, N, K = 2, 4, 512, 640
    A16 = bf16_normal((B, M, K), 1.0, 93)
    W16 = bf16_normal((B, N, K), 0.02, 94)
    assert spg.gemm_plan(M, N, K, "e4m3_tensor", "store", batch=B)["kernel"] == 3
    qa, sa = spg.quantize_tensor(dev(A16))
    qw, sw = spg.quantize_tensor(dev(W16))
    out = host_u16(spg.gemm_scaled(qa, sa, qw, sw, "store", fmt="e4m3_tensor"))
    for b in range(B):
        qao, sao = oracle.quantize_tensor(A16[b])
        qwo, swo = oracle.quantize_tensor(W16[b])
        D, Da = oracle.gemm_e4m3_sums(qao, qwo)
        y, S, _ = oracle.epilogue("store", D, Da, sao[0], swo[0])
        check_close(out[b], y, S, f"narrow per-batch weight {b}")


NARROW_NVFP4 = [((1, 64, 256), "store", "row"), ((5, 200, 1024), "add", "blocked"),
                ((16, 2060, 512), "swiglu", "row"), ((31, 520, 2048), "store", "blocked"),
                ((16, 5120, 6144), "add", "blocked"), ((16, 34816, 5120), "swiglu", "blocked"),
                ((33, 300, 1024), "store", "row"), ((64, 2048, 4096), "add", "blocked"),
                ((7, 400, 512), "swiglu", "row"), ((48, 520, 1056), "store", "row"),
                # decode-width kernel (K % 64 == 0): K tails inside a chunk,
                # two token blocks; K % 64 != 0 stays on the tiled route
                ((1, 1000, 1056), "store", "row"), ((20, 1034, 96), "swiglu", "row"),
                ((9, 520, 768), "add", "blocked"), ((32, 2048, 256), "add", "row"),
                ((16, 5120, 6144), "add", "row"), ((5, 1000, 320), "swiglu", "row"),
                ((3, 1024, 64), "store", "row")]


@pytest.mark.parametrize("shape,epi,layout", NARROW_NVFP4, ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_gemm_nvfp4_narrow(spg, shape, epi, layout):
    # few tokens on the NVFP4 path: one (<= 32 tokens) or two (<= 64) active
    # A blocks per wave, the weight-streaming K split, both scale-plane
    # layouts (K = 1056: the general path, row-major only)
    M, N, K = shape
    A16 = bf16_normal((M, K), 1.0, 170 + M)
    W16 = bf16_normal((N, K), 0.02, 171 + N)
    R16 = bf16_normal((M, N), 1.0, 172) if epi == "add" else None
    qa, bsa, ta = spg.quantize_block16(dev(A16), layout=layout)
    qw, bsw, tw = spg.quantize_block16(dev(W16), layout=layout)
    out = spg.gemm_scaled(qa, bsa, qw, bsw, epi, residual=dev(R16) if R16 is not None else None,
                          fmt="nvfp4", tscale_a=ta, tscale_w=tw, scale_layout=layout)
    ref = oracle_nvfp4(A16, W16, epi, R16)
    check_close(host_u16(out), ref["y"], ref["S"], f"nvfp4 narrow {shape} {epi} {layout}")


# ---------------------------------------------------------------------------
# padded leading dimensions: codes with row strides above K, output and
# residual with row strides above N (odd element strides for the bf16 ones);
# the padding of the output must stay untouched.  General tiles, split-K and
# the few-token instantiation.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,epi", [(300, 260, 320, "add"), (1000, 1030, 4096, "add"), (16, 520, 2080, "swiglu"),
                                       (130, 264, 512, "store"), (16, 1040, 2080, "swiglu"), (7, 600, 528, "add")])
def test_gemm_padded_leading_dimensions(spg, M, N, K, epi):
    A16 = bf16_normal((M, K), 1.0, M + 11)
    W16 = bf16_normal((N, K), 0.02, N + 13)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, M + 17) if epi == "add" else None
    qa_buf = torch.zeros((M, K + 32), dtype=torch.uint8, device="cuda")
    qw_buf = torch.zeros((N, K + 48), dtype=torch.uint8, device="cuda")
    sa = torch.empty(M, dtype=torch.float32, device="cuda")
    sw = torch.empty(N, dtype=torch.float32, device="cuda")
    spg.quantize_rowwise(dev(A16), out=qa_buf[:, :K], scale=sa)
    spg.quantize_rowwise(dev(W16), out=qw_buf[:, :K], scale=sw)
    out_buf = torch.full((M, n_out + 7), -7.0, dtype=torch.bfloat16, device="cuda")   # ldo odd
    res = None
    if R16 is not None:
        r_buf = torch.zeros((M, n_out + 5), dtype=torch.bfloat16, device="cuda")      # ldr odd
        r_buf[:, :n_out] = dev(R16)
        res = r_buf[:, :n_out]
    ws = spg.gemm_workspace(qa_buf[:, :K], qw_buf[:, :K], "e4m3_row", epi, out=out_buf[:, :n_out], residual=res)
    spg.gemm_scaled(qa_buf[:, :K], sa, qw_buf[:, :K], sw, epi, residual=res, out=out_buf[:, :n_out], workspace=ws)
    torch.cuda.synchronize()
    got = host_u16(out_buf)
    ref = oracle.linear_e4m3_rowwise(A16, W16, epi, R16)
    check_close(np.ascontiguousarray(got[:, :n_out]), ref["y"], ref["S"], f"padded {M}x{N}x{K} {epi}")
    pad = np.float32(-7.0).view(np.uint32) >> 16
    assert np.all(got[:, n_out:] == pad), "output padding written"


# ---------------------------------------------------------------------------
# the tail-exercising widths the pages test their ops at (ninfer PR #167:
# 1345, 1153, 4001 and 321 - widths that are not whole tiles), with canary
# guard bands around every output: quantized codes, scales and the GEMM
# output are written into the interior of larger buffers whose borders must
# keep their sentinel bytes.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,epi", [(321, 1345, 512, "store"), (1153, 321, 1040, "add"), (1345, 2 * 1153, 256, "swiglu"),
                                       (4001, 321, 128, "add"), (33, 4001, 2064, "store"),
                                       (16, 1345, 1040, "add"), (32, 2 * 1153, 256, "swiglu")])
def test_gemm_page_tail_widths_with_guard_bands(spg, M, N, K, epi):
    A16 = bf16_normal((M, K), 1.0, M * 3 + 1)
    W16 = bf16_normal((N, K), 0.02, N * 5 + 2)
    n_out = N // 2 if epi == "swiglu" else N
    R16 = bf16_normal((M, n_out), 1.0, M + N + 3) if epi == "add" else None
    G = 16                                                         # guard rows / columns
    qa_buf = torch.full((M + 2, K + G), 0xA5, dtype=torch.uint8, device="cuda")
    qw_buf = torch.full((N + 2, K + G), 0x5A, dtype=torch.uint8, device="cuda")
    sa_buf = torch.full((M + G,), -3.0, dtype=torch.float32, device="cuda")
    sw_buf = torch.full((N + G,), -5.0, dtype=torch.float32, device="cuda")
    qa, sa = qa_buf[1:M + 1, :K], sa_buf[4:M + 4]
    qw, sw = qw_buf[1:N + 1, :K], sw_buf[4:N + 4]
    spg.quantize_rowwise(dev(A16), out=qa, scale=sa)
    spg.quantize_rowwise(dev(W16), out=qw, scale=sw)
    out_buf = torch.full((M + 2, n_out + G), -7.0, dtype=torch.bfloat16, device="cuda")
    out = out_buf[1:M + 1, 8:8 + n_out]
    res = dev(R16) if R16 is not None else None
    spg.gemm_scaled(qa, sa, qw, sw, epi, residual=res, out=out)
    torch.cuda.synchronize()

    qa_h, qw_h = qa_buf.cpu().numpy(), qw_buf.cpu().numpy()
    qao, sao = oracle.quantize_rowwise(A16)
    qwo, swo = oracle.quantize_rowwise(W16)
    assert np.array_equal(qa_h[1:M + 1, :K], qao) and np.array_equal(qw_h[1:N + 1, :K], qwo)
    assert np.array_equal(sa.cpu().numpy().view(np.uint32), sao.view(np.uint32))
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), swo.view(np.uint32))
    qa_h[1:M + 1, :K] = 0xA5
    qw_h[1:N + 1, :K] = 0x5A
    assert np.all(qa_h == 0xA5) and np.all(qw_h == 0x5A), "code guard bands written"
    sa_h, sw_h = sa_buf.cpu().numpy(), sw_buf.cpu().numpy()
    assert np.all(np.delete(sa_h, np.s_[4:M + 4]) == -3.0) and np.all(np.delete(sw_h, np.s_[4:N + 4]) == -5.0)

    got = host_u16(out_buf)
    ref = oracle.linear_e4m3_rowwise(A16, W16, epi, R16)
    check_close(np.ascontiguousarray(got[1:M + 1, 8:8 + n_out]), ref["y"], ref["S"], f"widths {M}x{N}x{K} {epi}")
    sentinel = np.float32(-7.0).view(np.uint32) >> 16
    got[1:M + 1, 8:8 + n_out] = sentinel
    assert np.all(got == sentinel), "output guard band written"


def _interior(buf: torch.Tensor, off: int, n: int) -> torch.Tensor:
    return buf[off:off + n]


@pytest.mark.parametrize("M,N,K", [(321, 1345, 1024), (33, 300, 1056)])
def test_nvfp4_and_tensor_quantizers_and_gemm_with_guard_bands(spg, M, N, K):
    # quantize_block16 / quantize_tensor through the C ABI into the middle of
    # larger buffers, then the NVFP4 GEMM into the middle of a larger output;
    # every byte outside the written ranges must keep its sentinel
    G = 64
    A16 = bf16_normal((M, K), 1.0, M + 71)
    W16 = bf16_normal((N, K), 0.02, N + 72)
    outs = {}
    for name, x16 in (("a", A16), ("w", W16)):
        R = x16.shape[0]
        x = dev(x16)
        qbuf = torch.full((R * K // 2 + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
        sbuf = torch.full((R * K // 16 + 2 * G,), 0x5A, dtype=torch.uint8, device="cuda")
        tbuf = torch.full((2 * G // 4 + 1,), -9.0, dtype=torch.float32, device="cuda")
        nws = spg.lib.quantize_block16_workspace_bytes(R, K)
        ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
        q, bs, t = _interior(qbuf, G, R * K // 2), _interior(sbuf, G + 3, R * K // 16), _interior(tbuf, G // 4, 1)
        st = spg.lib.quantize_block16(spg._ptr(x), R, K, spg._ptr(q), spg._ptr(bs), spg._ptr(t), spg.SCALES_ROW_MAJOR,
                                      spg._ptr(ws), ws.numel(), spg._stream(x))
        assert st == 0
        torch.cuda.synchronize()
        qo, bso, to = oracle.quantize_block16(x16)
        assert np.array_equal(q.cpu().numpy(), qo.reshape(-1)) and np.array_equal(bs.cpu().numpy(), bso.reshape(-1))
        assert t.cpu().numpy().view(np.uint32)[0] == np.float32(to).view(np.uint32)
        qh, sh, th = qbuf.cpu().numpy(), sbuf.cpu().numpy(), tbuf.cpu().numpy()
        assert np.all(qh[:G] == 0xA5) and np.all(qh[G + R * K // 2:] == 0xA5)
        assert np.all(sh[:G + 3] == 0x5A) and np.all(sh[G + 3 + R * K // 16:] == 0x5A)
        assert np.all(np.delete(th, G // 4) == -9.0)
        outs[name] = (q.view(R, K // 2), bs.view(R, K // 16), t)
        # per-tensor FP8 of the same matrix, as a batch of one, into a guarded buffer
        qt_buf = torch.full((R * K + 2 * G,), 0x3C, dtype=torch.uint8, device="cuda")
        st_buf = torch.full((8,), -9.0, dtype=torch.float32, device="cuda")
        nws = spg.lib.quantize_tensor_workspace_bytes(1, R, K)
        ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
        qt, stt = _interior(qt_buf, G, R * K), _interior(st_buf, 4, 1)
        assert spg.lib.quantize_tensor(spg._ptr(x), 1, R, K, R * K, spg._ptr(qt), spg._ptr(stt), spg._ptr(ws),
                                       ws.numel(), spg._stream(x)) == 0
        torch.cuda.synchronize()
        qto, sto = oracle.quantize_tensor(x16)
        assert np.array_equal(qt.cpu().numpy(), qto.reshape(-1))
        assert st_buf.cpu().numpy().view(np.uint32)[4] == sto.view(np.uint32)[0]
        qth = qt_buf.cpu().numpy()
        assert np.all(qth[:G] == 0x3C) and np.all(qth[G + R * K:] == 0x3C)
        assert np.all(np.delete(st_buf.cpu().numpy(), 4) == -9.0)

    (qa, bsa, ta), (qw, bsw, tw) = outs["a"], outs["w"]
    out_buf = torch.full((M + 2, N + 16), -7.0, dtype=torch.bfloat16, device="cuda")
    out = out_buf[1:M + 1, 8:8 + N]
    spg.gemm_scaled(qa, bsa, qw, bsw, "store", fmt="nvfp4", tscale_a=ta, tscale_w=tw, out=out)
    torch.cuda.synchronize()
    got = host_u16(out_buf)
    ref = oracle_nvfp4(A16, W16, "store")
    check_close(np.ascontiguousarray(got[1:M + 1, 8:8 + N]), ref["y"], ref["S"], f"nvfp4 guard {M}x{N}x{K}")
    sentinel = np.float32(-7.0).view(np.uint32) >> 16
    got[1:M + 1, 8:8 + N] = sentinel
    assert np.all(got == sentinel), "NVFP4 output guard band written"
