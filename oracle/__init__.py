"""CPU oracle for the scaled low-precision GEMM path (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never does, and
the two share no code.  The arithmetic lives in ``oracle.c`` (plain C, fp64
accumulation, IEEE binary32 where the method rounds to fp32); this module only
marshals numpy arrays and composes the C steps in the order the pages give:
quantize, multiply the decoded codes exactly, scale, apply the epilogue, round
once to bf16.

Arrays of bf16 values are carried as ``np.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

STORE, ADD, SWIGLU = 0, 1, 2
EPILOGUES = {"store": STORE, "add": ADD, "swiglu": SWIGLU}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (OpenMP, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", "-ffp-contract=off", "-fvisibility=hidden",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    lib = ctypes.CDLL(build())
    c_i64, c_f, c_d, c_u32, c_p = (ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                   ctypes.c_uint32, ctypes.c_void_p)
    sig = {
        "spo_threads": (ctypes.c_int, []),
        "spo_bf16_to_f32": (c_f, [ctypes.c_uint16]),
        "spo_bf16_from_f64": (ctypes.c_uint16, [c_d]),
        "spo_e4m3_value": (c_d, [c_u32]),
        "spo_e2m1_value": (c_d, [c_u32]),
        "spo_e4m3_encode": (c_u32, [c_f]),
        "spo_e2m1_encode": (c_u32, [c_f]),
        "spo_quantize_rowwise": (None, [c_p, c_i64, c_i64, c_i64, c_p, c_i64, c_p]),
        "spo_amax_bf16": (c_f, [c_p, c_i64, c_i64, c_i64]),
        "spo_quantize_tensor": (None, [c_p, c_i64, c_i64, c_i64, c_i64, c_p, c_p]),
        "spo_quantize_rows_with_scale": (None, [c_p, c_i64, c_i64, c_i64, c_p, c_i64, c_p, c_i64]),
        "spo_nvfp4_tensor_scale": (c_f, [c_p, c_i64, c_i64, c_i64]),
        "spo_quantize_block16_rows": (None, [c_p, c_i64, c_i64, c_i64, c_f, c_p, c_p]),
        "spo_quantize_block16": (None, [c_p, c_i64, c_i64, c_i64, c_p, c_p, c_p]),
        "spo_gemm_e4m3": (None, [c_p, c_i64, c_p, c_i64, c_i64, c_i64, c_i64, c_p, c_p]),
        "spo_gemm_nvfp4": (None, [c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_p, c_p]),
        "spo_epilogue": (None, [ctypes.c_int, c_p, c_p, c_i64, c_i64, c_p, c_p, c_p, c_i64,
                                c_p, c_p, c_p, c_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_lib.spo_threads())


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    assert x.dtype == np.uint16, "bf16 inputs are carried as uint16 bit patterns"
    return x


# --------------------------------------------------------------------------
# scalar format helpers
# --------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return _lib.spo_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    return _lib.spo_e2m1_value(int(code))


def e4m3_encode(v: float) -> int:
    return _lib.spo_e4m3_encode(float(np.float32(v)))


def e2m1_encode(v: float) -> int:
    return _lib.spo_e2m1_encode(float(np.float32(v)))


def bf16_from_f64(y: float) -> int:
    return _lib.spo_bf16_from_f64(float(y))


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    return (np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# quantizers
# --------------------------------------------------------------------------

def quantize_rowwise(x: np.ndarray):
    """Per-row E4M3: returns (codes u8 [R,K], scales f32 [R])."""
    x = _u16(x)
    R, K = x.shape
    q = np.empty((R, K), np.uint8)
    s = np.empty(R, np.float32)
    _lib.spo_quantize_rowwise(_p(x), R, K, K, _p(q), K, _p(s))
    return q, s


def quantize_tensor(x: np.ndarray):
    """Per-matrix E4M3 for x of shape [R,K] or [B,R,K]: (codes, scales [B])."""
    x = _u16(x)
    xb = x.reshape((-1,) + x.shape[-2:])
    B, R, K = xb.shape
    q = np.empty(xb.shape, np.uint8)
    s = np.empty(B, np.float32)
    _lib.spo_quantize_tensor(_p(xb), B, R, K, R * K, _p(q), _p(s))
    return q.reshape(x.shape), s


def amax(x: np.ndarray) -> np.float32:
    x = _u16(x).reshape(-1, x.shape[-1])
    return np.float32(_lib.spo_amax_bf16(_p(x), x.shape[0], x.shape[1], x.shape[1]))


def quantize_rows_with_scale(x: np.ndarray, scale) -> np.ndarray:
    """E4M3 codes of rows x [R,K] under given scales (array [R] or a scalar)."""
    x = _u16(x)
    R, K = x.shape
    sc = np.ascontiguousarray(np.atleast_1d(np.asarray(scale, np.float32)))
    stride = 0 if sc.size == 1 else 1
    assert stride == 0 or sc.size == R
    q = np.empty((R, K), np.uint8)
    _lib.spo_quantize_rows_with_scale(_p(x), R, K, K, _p(sc), stride, _p(q), K)
    return q


def nvfp4_tensor_scale(x: np.ndarray) -> np.float32:
    x = _u16(x)
    return np.float32(_lib.spo_nvfp4_tensor_scale(_p(x), x.shape[0], x.shape[1], x.shape[1]))


def quantize_block16_rows(x: np.ndarray, t) -> tuple[np.ndarray, np.ndarray]:
    x = _u16(x)
    R, K = x.shape
    assert K % 16 == 0
    q = np.empty((R, K // 2), np.uint8)
    bs = np.empty((R, K // 16), np.uint8)
    _lib.spo_quantize_block16_rows(_p(x), R, K, K, float(np.float32(t)), _p(q), _p(bs))
    return q, bs


def quantize_block16(x: np.ndarray):
    """NVFP4: (codes u8 [R,K/2], block scales u8 [R,K/16], tensor scale f32)."""
    x = _u16(x)
    R, K = x.shape
    assert K % 16 == 0
    q = np.empty((R, K // 2), np.uint8)
    bs = np.empty((R, K // 16), np.uint8)
    t = np.empty(1, np.float32)
    _lib.spo_quantize_block16(_p(x), R, K, K, _p(q), _p(bs), _p(t))
    return q, bs, t[0]


# --------------------------------------------------------------------------
# GEMM + epilogue
# --------------------------------------------------------------------------

def gemm_e4m3_sums(Aq: np.ndarray, Wq: np.ndarray):
    """Exact D = dec(A) dec(W)^T and sum of |products| (both fp64 [M,N])."""
    Aq = np.ascontiguousarray(Aq, np.uint8)
    Wq = np.ascontiguousarray(Wq, np.uint8)
    M, K = Aq.shape
    N, K2 = Wq.shape
    assert K == K2
    D = np.empty((M, N), np.float64)
    Da = np.empty((M, N), np.float64)
    _lib.spo_gemm_e4m3(_p(Aq), K, _p(Wq), K, M, N, K, _p(D), _p(Da))
    return D, Da


def gemm_nvfp4_sums(Aq, As, Wq, Ws):
    Aq, As, Wq, Ws = (np.ascontiguousarray(a, np.uint8) for a in (Aq, As, Wq, Ws))
    M, Kh = Aq.shape
    N = Wq.shape[0]
    K = 2 * Kh
    assert Wq.shape == (N, Kh) and As.shape == (M, K // 16) and Ws.shape == (N, K // 16)
    D = np.empty((M, N), np.float64)
    Da = np.empty((M, N), np.float64)
    _lib.spo_gemm_nvfp4(_p(Aq), _p(As), _p(Wq), _p(Ws), M, N, K, _p(D), _p(Da))
    return D, Da


def bias_e4m3(codes: np.ndarray, scale) -> np.ndarray:
    """A bias stored as E4M3 codes with one fp32 scale, dequantized: the exact
    fp64 values dec(code) * scale (AstrAI commit log, the commit fusing the
    bias: a non-null bias scale means FP8 storage dequantized in the
    epilogue)."""
    c = np.asarray(codes, dtype=np.uint8)
    return E4M3_TABLE[c] * np.float64(np.float32(scale))


def epilogue(epi, D, Dabs, ascale, wscale, residual=None, bias=None):
    """Apply scales and the epilogue in fp64; returns (y, S, out_bf16_bits).
    ADD takes a bf16 residual [M, Nout] and/or `bias`, fp64 values [Nout]
    added to every row after the operand scales, before the one rounding."""
    epi = EPILOGUES.get(epi, epi)
    D = np.ascontiguousarray(D, np.float64)
    Dabs = np.ascontiguousarray(Dabs, np.float64)
    M, Nw = D.shape
    a = np.ascontiguousarray(np.broadcast_to(np.asarray(ascale, np.float64), (M,)))
    w = np.ascontiguousarray(np.broadcast_to(np.asarray(wscale, np.float64), (Nw,)))
    if epi == SWIGLU:
        assert Nw % 2 == 0
    Nout = Nw // 2 if epi == SWIGLU else Nw
    rp, ldr, bp = None, 0, None
    if epi == ADD:
        assert residual is not None or bias is not None
        if residual is not None:
            r = _u16(residual)
            assert r.shape == (M, Nout)
            rp, ldr = _p(r), Nout
        if bias is not None:
            b = np.ascontiguousarray(bias, np.float64)
            assert b.shape == (Nout,)
            bp = _p(b)
    else:
        assert residual is None and bias is None
    y = np.empty((M, Nout), np.float64)
    S = np.empty((M, Nout), np.float64)
    out = np.empty((M, Nout), np.uint16)
    _lib.spo_epilogue(int(epi), _p(D), _p(Dabs), M, Nw, _p(a), _p(w), rp, ldr, bp,
                      _p(y), _p(S), _p(out))
    return y, S, out


def linear_e4m3_rowwise(A_bf16, W_bf16, epi, residual=None, bias=None):
    """Whole path, row-scaled FP8: quantize both operands per row, exact GEMM,
    scales, epilogue.  Returns dict with codes, scales, y, S, out."""
    Aq, sa = quantize_rowwise(A_bf16)
    Wq, sw = quantize_rowwise(W_bf16)
    D, Da = gemm_e4m3_sums(Aq, Wq)
    y, S, out = epilogue(epi, D, Da, sa, sw, residual, bias)
    return dict(Aq=Aq, sa=sa, Wq=Wq, sw=sw, y=y, S=S, out=out)


def within_tolerance(gpu_bf16_bits: np.ndarray, y: np.ndarray, S: np.ndarray):
    """Acceptance bound per element: |gpu - y| <= 2^-8 |y| + 2^-12 S + 2^-134,
    gpu finite.  The last term is half of bf16's smallest step (2^-133, the
    spacing of its subnormals): below bf16's normal range the output format
    cannot come closer to y than that, and with it the correctly rounded
    result passes at every magnitude.  Returns (ok_mask, excess) where
    excess = |err| / bound."""
    g = bf16_to_f64(gpu_bf16_bits)
    bound = 2.0 ** -8 * np.abs(y) + 2.0 ** -12 * S + 2.0 ** -134
    err = np.abs(g - y)
    ok = np.isfinite(g) & (err <= bound)
    with np.errstate(divide="ignore", invalid="ignore"):
        excess = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    return ok, excess
