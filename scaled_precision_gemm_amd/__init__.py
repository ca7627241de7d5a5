"""Python binding of the gfx950 scaled low-precision GEMM library.

Argument marshalling only: each function checks dtypes and shapes, allocates
outputs with torch on the input's device (torch is the memory and stream
provider), and calls the C ABI of ``libspg.so`` (declared in
``include/spg.h``) on torch's current stream.  Every step of the path runs in
the library's HIP kernels; there is no fallback.  Importing this package
fails loudly when the library is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "quantize_rowwise", "quantize_tensor", "quantize_block16", "gemm_scaled",
    "gemm_plan", "gemm_workspace", "route_select", "route_cost", "probe_mfma", "probe_read", "probe_fp4_rounding",
    "lib", "LIB_PATH",
    "FMT_E4M3_ROW", "FMT_E4M3_TENSOR", "FMT_NVFP4", "EPI_STORE", "EPI_ADD", "EPI_SWIGLU",
    "SpgError", "check_operands", "block16_scale_shape", "SCALES_ROW_MAJOR", "SCALES_BLOCKED", "QUANT_SINGLE_LAUNCH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspg.so")

FMT_E4M3_ROW, FMT_E4M3_TENSOR, FMT_NVFP4 = 0, 1, 2
EPI_STORE, EPI_ADD, EPI_SWIGLU = 0, 1, 2
SCALES_ROW_MAJOR, SCALES_BLOCKED = 0, 1
QUANT_SINGLE_LAUNCH = 0x100
_LAYOUT = {"row": SCALES_ROW_MAJOR, "blocked": SCALES_BLOCKED}
_EPI = {"store": EPI_STORE, "add": EPI_ADD, "swiglu": EPI_SWIGLU}
_FMT = {"e4m3_row": FMT_E4M3_ROW, "e4m3_tensor": FMT_E4M3_TENSOR, "nvfp4": FMT_NVFP4}


class SpgError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {lib.spg_status_string(status).decode()} (status {status})")
        self.status = status


MAX_OUT_SPLITS = 8
LAYOUT_NT, LAYOUT_A_KMAJOR, LAYOUT_W_KMAJOR = 0, 1, 2


class OutSplit(ctypes.Structure):
    _fields_ = [
        ("count", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("col_end", ctypes.c_int64 * MAX_OUT_SPLITS), ("out", ctypes.c_void_p * MAX_OUT_SPLITS),
        ("ldo", ctypes.c_int64 * MAX_OUT_SPLITS), ("stride_o", ctypes.c_int64 * MAX_OUT_SPLITS),
    ]


class GemmDesc(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("batch", ctypes.c_int64),
        ("lda", ctypes.c_int64), ("ldw", ctypes.c_int64), ("ldo", ctypes.c_int64), ("ldr", ctypes.c_int64),
        ("stride_a", ctypes.c_int64), ("stride_w", ctypes.c_int64),
        ("stride_o", ctypes.c_int64), ("stride_r", ctypes.c_int64),
        ("format", ctypes.c_int32), ("scale_layout", ctypes.c_int32),
        ("tscale_a", ctypes.c_void_p), ("tscale_w", ctypes.c_void_p),
        ("clock_probe", ctypes.c_void_p), ("bias_scale", ctypes.c_void_p),
        ("out_split", ctypes.POINTER(OutSplit)), ("layout", ctypes.c_int32), ("reserved2", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [
        ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32), ("split_k", ctypes.c_int32),
        ("tiles", ctypes.c_int64), ("workgroups", ctypes.c_int64), ("kernel", ctypes.c_int32),
        ("tail_split", ctypes.c_int32), ("tail_tiles", ctypes.c_int64),
        ("tail_bm", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class RouteCandidate(ctypes.Structure):
    _fields_ = [("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("per_unit", ctypes.c_int32),
                ("factor", ctypes.c_double)]


# Exported symbols and their signatures (mirrors include/spg.h).
_P, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
SIGNATURES = {
    "spg_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "quantize_rowwise": (ctypes.c_int, [_P, _I64, _I64, _I64, _P, _I64, _P, _P]),
    "quantize_tensor_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "quantize_tensor": (ctypes.c_int, [_P, _I64, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "quantize_block16_workspace_bytes": (_SZ, [_I64, _I64]),
    "quantize_block16_path": (ctypes.c_int, [_I64, _I64]),
    "quantize_block16": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, ctypes.c_int, _P, _SZ, _P]),
    "quantize_block16_noalloc": (ctypes.c_int, [_P, _I64, _I64, _P, _P, _P, ctypes.c_int, _P]),
    "spg_gemm_desc_init": (None, [ctypes.POINTER(GemmDesc), _I64, _I64, _I64, _I32]),
    "gemm_scaled_workspace_bytes": (_SZ, [ctypes.POINTER(GemmDesc), ctypes.c_int]),
    "gemm_scaled": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, ctypes.c_int, ctypes.POINTER(GemmDesc), _P, _SZ, _P]),
    "spg_route_cost": (ctypes.c_double, [ctypes.POINTER(RouteCandidate), _I64, _I64, _I64, _I32]),
    "spg_route_select": (ctypes.c_int, [ctypes.POINTER(RouteCandidate), _I32, _I64, _I64, _I64, _I32]),
    "spg_gemm_plan": (ctypes.c_int, [ctypes.POINTER(GemmDesc), ctypes.c_int, _I32, ctypes.POINTER(Plan)]),
    "spg_probe_mfma": (ctypes.c_int, [ctypes.c_int, _I64, _I32, _P, _P, _P]),
    "spg_probe_read": (ctypes.c_int, [_P, _I64, _I32, _P, _P]),
    "spg_probe_fp4_rounding": (ctypes.c_int, [_P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run scaled_precision_gemm_amd/build.py (hipcc, gfx950)")
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


lib = _load()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    """torch's current stream on t's device, as a raw hipStream_t value."""
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(status: int, what: str):
    if status != 0:
        raise SpgError(status, what)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

def quantize_rowwise(x: torch.Tensor, out: torch.Tensor | None = None, scale: torch.Tensor | None = None):
    """Per-row E4M3: x bf16 [R, K] -> (codes uint8 [R, K], scales fp32 [R])."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_cuda, "x must be a 2-D bf16 CUDA tensor")
    _need(x.stride(1) == 1, "x rows must be contiguous")
    R, K = x.shape
    q = out if out is not None else torch.empty((R, K), dtype=torch.uint8, device=x.device)
    s = scale if scale is not None else torch.empty((R,), dtype=torch.float32, device=x.device)
    _check(lib.quantize_rowwise(_ptr(x), R, K, x.stride(0), _ptr(q), q.stride(0), _ptr(s), _stream(x)),
           "quantize_rowwise")
    return q, s


def quantize_tensor(x: torch.Tensor):
    """Per-matrix E4M3: x bf16 [R, K] or [B, R, K] -> (codes, scales fp32 [B])."""
    _need(x.dtype == torch.bfloat16 and x.dim() in (2, 3) and x.is_cuda and x.is_contiguous(),
          "x must be a contiguous 2-D or 3-D bf16 CUDA tensor")
    xb = x.unsqueeze(0) if x.dim() == 2 else x
    B, R, K = xb.shape
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = torch.empty((B,), dtype=torch.float32, device=x.device)
    nws = lib.quantize_tensor_workspace_bytes(B, R, K)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=x.device)
    _check(lib.quantize_tensor(_ptr(xb), B, R, K, R * K, _ptr(q), _ptr(s), _ptr(ws), ws.numel(), _stream(x)),
           "quantize_tensor")
    return q, s


def block16_scale_shape(R: int, K: int, layout="row") -> tuple:
    """Shape of the NVFP4 block-scale plane: [R, K/16] row-major, or the
    blocked plane of ceil(R/256) row tiles x K/256 stages x 4096 bytes."""
    if _LAYOUT.get(layout, layout) == SCALES_BLOCKED:
        return ((R + 255) // 256, K // 256, 4096)
    return (R, K // 16)


def quantize_block16(x: torch.Tensor, layout="row", single_launch=False):
    """NVFP4: x bf16 [R, K] -> (codes uint8 [R, K/2], block scales uint8
    (E4M3; [R, K/16] row-major, or the blocked plane of block16_scale_shape),
    tensor scale fp32 [1]).  single_launch requests the one-launch quantizer
    (same results)."""
    _need(x.dtype == torch.bfloat16 and x.dim() == 2 and x.is_cuda and x.is_contiguous(),
          "x must be a contiguous 2-D bf16 CUDA tensor")
    lay = _LAYOUT.get(layout, layout)
    R, K = x.shape
    q = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
    bs = torch.empty(block16_scale_shape(R, K, lay), dtype=torch.uint8, device=x.device)
    t = torch.empty((1,), dtype=torch.float32, device=x.device)
    nws = lib.quantize_block16_workspace_bytes(R, K)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=x.device)
    flags = lay | (QUANT_SINGLE_LAUNCH if single_launch else 0)
    _check(lib.quantize_block16(_ptr(x), R, K, _ptr(q), _ptr(bs), _ptr(t), flags, _ptr(ws), ws.numel(), _stream(x)),
           "quantize_block16")
    return q, bs, t


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _desc(fmt: int, M: int, N: int, K: int) -> GemmDesc:
    d = GemmDesc()
    lib.spg_gemm_desc_init(ctypes.byref(d), M, N, K, fmt)
    return d


def _logical_dims(A, W, a_kmajor, w_kmajor):
    """(M, N, K in code bytes) of the product from the stored operands: A is
    [M, K] or, K-major, [K, M]; W is [N, K] or, K-major, [K, N]."""
    M, Ka = (A.shape[-1], A.shape[-2]) if a_kmajor else (A.shape[-2], A.shape[-1])
    N, Kw = (W.shape[-1], W.shape[-2]) if w_kmajor else (W.shape[-2], W.shape[-1])
    return M, N, Ka, Kw


def make_desc(A: torch.Tensor, W: torch.Tensor, fmt, epilogue, out=None, residual=None,
              tscale_a=None, tscale_w=None, a_kmajor=False, w_kmajor=False) -> tuple[GemmDesc, int, int]:
    fmt = _FMT.get(fmt, fmt)
    epi = _EPI.get(epilogue, epilogue)
    _need(A.dtype == torch.uint8 and W.dtype == torch.uint8, "A and W must be uint8 code tensors")
    batched = A.dim() == 3 or W.dim() == 3
    A3 = A if A.dim() == 3 else A.unsqueeze(0)
    W3 = W if W.dim() == 3 else W.unsqueeze(0)
    _need(A3.stride(2) == 1 and W3.stride(2) == 1, "rows must be contiguous")
    batch = max(A3.shape[0], W3.shape[0])
    _need(A3.shape[0] in (1, batch) and W3.shape[0] in (1, batch), "batch sizes must match or be 1")
    M, N, Kc, Kw = _logical_dims(A3, W3, a_kmajor, w_kmajor)
    K = 2 * Kc if fmt == FMT_NVFP4 else Kc
    _need(Kw == Kc, "A and W disagree on K")
    d = _desc(fmt, M, N, K)
    d.layout = (LAYOUT_A_KMAJOR if a_kmajor else 0) | (LAYOUT_W_KMAJOR if w_kmajor else 0)
    d.batch = batch
    d.lda, d.ldw = A3.stride(1), W3.stride(1)
    d.stride_a = A3.stride(0) if A3.shape[0] > 1 else 0
    d.stride_w = W3.stride(0) if W3.shape[0] > 1 else 0
    n_out = N // 2 if epi == EPI_SWIGLU else N
    if out is not None:
        o3 = out if out.dim() == 3 else out.unsqueeze(0)
        d.ldo = o3.stride(1)
        d.stride_o = o3.stride(0) if batch > 1 else 0
    else:
        d.ldo = n_out
        d.stride_o = M * n_out if batch > 1 else 0
    if residual is not None and residual.dim() == 1:
        # one row [N]: a bias added to every token row of every batch entry
        _need(residual.shape[0] == n_out and residual.stride(0) == 1, "a bias row must be contiguous [N]")
        d.ldr, d.stride_r = 0, 0
    elif residual is not None:
        r3 = residual if residual.dim() == 3 else residual.unsqueeze(0)
        d.ldr = r3.stride(1)
        d.stride_r = r3.stride(0) if r3.shape[0] > 1 else 0
    if fmt == FMT_NVFP4:
        d.tscale_a = tscale_a.data_ptr() if tscale_a is not None else None
        d.tscale_w = tscale_w.data_ptr() if tscale_w is not None else None
    return d, epi, batched


def check_out_split(segs, M, n_out, batch, batched, dev):
    """The segments of a split output: bf16 tensors [M, w] ([B, M, w] when
    batched), rows contiguous, 16-byte aligned with a row stride that is a
    multiple of 8, widths adding up to the output width with every boundary
    but the last a multiple of 64."""
    _need(isinstance(segs, (list, tuple)) and 1 <= len(segs) <= MAX_OUT_SPLITS,
          f"out_split takes 1 to {MAX_OUT_SPLITS} output tensors")
    end = 0
    for i, t in enumerate(segs):
        _need(isinstance(t, torch.Tensor) and t.device == dev and t.dtype == torch.bfloat16,
              f"output segment {i} must be a bf16 tensor on {dev}")
        _need(t.dim() == (3 if batched else 2), f"output segment {i} must be {'3' if batched else '2'}-D")
        _need(t.shape[-2] == M and (not batched or t.shape[0] == batch), f"output segment {i} has the wrong rows")
        _need(t.stride(-1) == 1 and t.stride(-2) % 8 == 0 and t.data_ptr() % 16 == 0,
              f"output segment {i}: contiguous rows, 16-byte aligned, row stride a multiple of 8")
        end += t.shape[-1]
        _need(t.shape[-1] > 0 and (i + 1 == len(segs) or end % 64 == 0),
              "every output segment boundary but the last must be a multiple of 64 columns")
    _need(end == n_out, f"the output segments must add up to {n_out} columns")


def check_operands(A, sa, W, sw, fmt, epilogue, out=None, residual=None, tscale_a=None, tscale_w=None,
                   scale_layout="row", bias_scale=None, out_split=None, a_kmajor=False, w_kmajor=False):
    """Shapes, dtypes, strides and devices of a gemm_scaled call, checked
    before anything reaches the library (raises ValueError).  The library
    trusts the sizes it is given, so an output, residual or scale tensor
    smaller than the descriptor says would be read or written out of
    bounds."""
    fmt = _FMT.get(fmt, fmt)
    epi = _EPI.get(epilogue, epilogue)
    _need(fmt in (FMT_E4M3_ROW, FMT_E4M3_TENSOR, FMT_NVFP4), f"unknown format {fmt}")
    _need(epi in (EPI_STORE, EPI_ADD, EPI_SWIGLU), f"unknown epilogue {epilogue}")
    _need(isinstance(A, torch.Tensor) and isinstance(W, torch.Tensor), "A and W must be tensors")
    _need(A.dtype == torch.uint8 and W.dtype == torch.uint8, "A and W must be uint8 code tensors")
    _need(A.dim() in (2, 3) and W.dim() in (2, 3), "A and W must be 2-D or 3-D")
    _need(A.stride(-1) == 1 and W.stride(-1) == 1, "rows of A and W must be contiguous")
    dev = A.device
    for name, t in (("W", W), ("sa", sa), ("sw", sw), ("out", out), ("residual", residual),
                    ("tscale_a", tscale_a), ("tscale_w", tscale_w), ("bias_scale", bias_scale)):
        _need(t is None or (isinstance(t, torch.Tensor) and t.device == dev), f"{name} must be on {dev}")
    Ab = A.shape[0] if A.dim() == 3 else 1
    Wb = W.shape[0] if W.dim() == 3 else 1
    batch = max(Ab, Wb)
    _need(Ab in (1, batch) and Wb in (1, batch), "batch sizes of A and W must match or be 1")
    batched = A.dim() == 3 or W.dim() == 3
    _need(fmt != FMT_NVFP4 or not (a_kmajor or w_kmajor), "K-major operands are taken only by the FP8 formats")
    M, N, Kc, Kw = _logical_dims(A, W, a_kmajor, w_kmajor)
    _need(Kw == Kc, "A and W disagree on K")
    for name, t, km in (("A", A, a_kmajor), ("W", W, w_kmajor)):
        _need(not km or (t.stride(-2) % 16 == 0 and t.data_ptr() % 16 == 0),
              f"a K-major {name} needs 16-byte aligned rows")
    n_out = N // 2 if epi == EPI_SWIGLU else N
    _need(sa is not None and sw is not None, "sa and sw are required")
    if fmt == FMT_E4M3_ROW:
        _need(sa.dtype == torch.float32 and sw.dtype == torch.float32, "row scales must be fp32")
        _need(sa.is_contiguous() and sa.numel() == Ab * M, f"sa must hold {Ab * M} fp32 row scales")
        _need(sw.is_contiguous() and sw.numel() == Wb * N, f"sw must hold {Wb * N} fp32 row scales")
    elif fmt == FMT_E4M3_TENSOR:
        _need(sa.dtype == torch.float32 and sw.dtype == torch.float32, "tensor scales must be fp32")
        _need(sa.is_contiguous() and sa.numel() == Ab, f"sa must hold {Ab} fp32 tensor scale(s)")
        _need(sw.is_contiguous() and sw.numel() == Wb, f"sw must hold {Wb} fp32 tensor scale(s)")
    else:
        _need(not batched, "NVFP4 takes one product (2-D operands)")
        _need(sa.dtype == torch.uint8 and sw.dtype == torch.uint8, "NVFP4 block scales are uint8 E4M3 codes")
        lay = _LAYOUT.get(scale_layout, scale_layout)
        _need(lay in (SCALES_ROW_MAJOR, SCALES_BLOCKED), f"unknown scale layout {scale_layout}")
        _need(lay == SCALES_ROW_MAJOR or (2 * Kc) % 256 == 0, "blocked scale planes need K % 256 == 0")
        sa_shape, sw_shape = block16_scale_shape(M, 2 * Kc, lay), block16_scale_shape(N, 2 * Kc, lay)
        _need(tuple(sa.shape) == sa_shape and sa.is_contiguous(), f"sa must be a contiguous {sa_shape} plane")
        _need(tuple(sw.shape) == sw_shape and sw.is_contiguous(), f"sw must be a contiguous {sw_shape} plane")
        for name, t in (("tscale_a", tscale_a), ("tscale_w", tscale_w)):
            _need(t is not None and t.dtype == torch.float32 and t.numel() == 1, f"{name} must be one fp32 value")
    if out is not None:
        want = (batch, M, n_out) if batched else (M, n_out)
        _need(out.dtype == torch.bfloat16, "out must be bf16")
        _need(tuple(out.shape) == want, f"out must have shape {want}")
        _need(out.stride(-1) == 1, "rows of out must be contiguous")
    if out_split is not None:
        _need(out is None, "out and out_split are exclusive")
        segs = list(out_split)
        if segs and all(isinstance(w, int) for w in segs):
            _need(len(segs) <= MAX_OUT_SPLITS and all(w > 0 for w in segs) and sum(segs) == n_out,
                  f"out_split widths: 1 to {MAX_OUT_SPLITS} positive widths adding up to {n_out}")
            _need(all(sum(segs[:i + 1]) % 64 == 0 for i in range(len(segs) - 1)),
                  "every output segment boundary but the last must be a multiple of 64 columns")
        else:
            check_out_split(segs, M, n_out, batch, batched, dev)
    if bias_scale is not None:
        # an E4M3 bias row: uint8 codes [N], one fp32 scale
        _need(epi == EPI_ADD, "a bias scale is taken only by the add epilogue")
        _need(bias_scale.dtype == torch.float32 and bias_scale.numel() == 1, "bias_scale must be one fp32 value")
        _need(residual is not None and residual.dtype == torch.uint8 and residual.dim() == 1
              and residual.shape[0] == n_out and residual.stride(0) == 1,
              f"with a bias scale the residual must be contiguous uint8 E4M3 codes [{n_out}]")
    elif epi == EPI_ADD:
        _need(residual is not None, "the add epilogue needs a residual")
        _need(residual.dtype == torch.bfloat16, "residual must be bf16")
        _need(residual.stride(-1) == 1, "rows of the residual must be contiguous")
        shapes = [(n_out,), (M, n_out)] + ([(batch, M, n_out), (1, M, n_out)] if batched else [])
        _need(tuple(residual.shape) in shapes, f"residual must have one of the shapes {shapes}")
    else:
        _need(residual is None, "a residual is taken only by the add epilogue")
    return fmt, epi


def gemm_scaled(A, sa, W, sw, epilogue="store", residual=None, fmt="e4m3_row",
                out=None, tscale_a=None, tscale_w=None, workspace=None, clock_probe=None, scale_layout="row",
                bias_scale=None, out_split=None, a_kmajor=False, w_kmajor=False):
    """out = epilogue(scale * A W^T) in bf16.

    e4m3_row: A uint8 [M,K], sa fp32 [M]; W uint8 [N,K], sw fp32 [N]
    e4m3_tensor: A [B,M,K] or [M,K], sa fp32 [B]; W likewise, sw fp32 [B]
    nvfp4: A uint8 [M,K/2], sa uint8 [M,K/16]; W [N,K/2], sw [N,K/16];
           tscale_a, tscale_w fp32 [1]; scale_layout "row" or "blocked" (both
           planes, as quantize_block16 wrote them)
    clock_probe: optional int64 tensor of 4 elements on the same device; the
           main GEMM launch records its clock counters there (see
           spg_gemm_desc.clock_probe): shader clock in GHz =
           (c[1] - c[0]) / (c[3] - c[2]) / 10
    bias_scale: optional fp32 [1] on the same device; with "add" and a
           residual of uint8 E4M3 codes [N], the bias added to every row is
           dec(code) * bias_scale (see spg_gemm_desc.bias_scale); without it
           a 1-D residual is a bf16 bias row
    out_split: optional list of output column widths (ints) or of bf16
           output tensors, one per column segment (see spg_out_split): the
           output goes to them instead of one tensor, and they are returned
           as a list (out must then be None)
    a_kmajor, w_kmajor: the operand is stored K-major - A as [K, M], W as
           [K, N] ([B, K, .] batched), as the backward products read them
           (dX = dY W: w_kmajor; dW = dY^T X: both); FP8 formats only
    """
    segs = None
    if out_split is None:
        # the checks and the descriptor depend only on what _sig reads, so a
        # call that repeats an earlier call's signature reuses its checked
        # descriptor (the per-call pointers are filled in below)
        try:
            key = (fmt, epilogue, scale_layout, a_kmajor, w_kmajor, _sig(A), _sig(sa), _sig(W), _sig(sw),
                   _sig(out), _sig(residual), _sig(tscale_a), _sig(tscale_w), _sig(bias_scale))
            hit = _GEMM_CACHE.get(key)
        except TypeError:      # a non-tensor argument or an unhashable option: the full checks report it
            key = hit = None
        if hit is None:
            hit = _prepare(A, sa, W, sw, fmt, epilogue, out, residual, tscale_a, tscale_w, scale_layout,
                           bias_scale, a_kmajor, w_kmajor)
            if key is not None:
                if len(_GEMM_CACHE) >= _GEMM_CACHE_MAX:
                    _GEMM_CACHE.clear()
                _GEMM_CACHE[key] = hit
        tmpl, epi, out_shape, nws = hit
        d = GemmDesc.from_buffer_copy(tmpl)
    else:
        check_operands(A, sa, W, sw, fmt, epilogue, out, residual, tscale_a, tscale_w, scale_layout, bias_scale,
                       out_split, a_kmajor, w_kmajor)
        _need(A.is_cuda, "operands must be CUDA tensors")
        d, epi, batched = make_desc(A, W, fmt, epilogue, out, residual, tscale_a, tscale_w, a_kmajor, w_kmajor)
        d.scale_layout = _LAYOUT.get(scale_layout, scale_layout)
        segs = list(out_split)
        if all(isinstance(w, int) for w in segs):
            # row strides rounded up to 8 elements (the library's alignment rule)
            segs = [torch.empty((d.batch, d.M, (w + 7) // 8 * 8) if batched else (d.M, (w + 7) // 8 * 8),
                                dtype=torch.bfloat16, device=A.device)[..., :w] for w in segs]
        split = OutSplit()
        split.count = len(segs)
        end = 0
        for i, t in enumerate(segs):
            end += t.shape[-1]
            split.col_end[i] = end
            split.out[i] = t.data_ptr()
            split.ldo[i] = t.stride(-2)
            split.stride_o[i] = t.stride(0) if batched else 0
        d.out_split = ctypes.pointer(split)
        out_shape = None
        nws = lib.gemm_scaled_workspace_bytes(ctypes.byref(d), epi)
    if clock_probe is not None:
        _need(isinstance(clock_probe, torch.Tensor) and clock_probe.dtype == torch.int64 and clock_probe.numel() == 4
              and clock_probe.is_contiguous() and clock_probe.device == A.device,
              "clock_probe must be 4 contiguous int64 values on A's device")
    if tscale_a is not None:
        d.tscale_a = tscale_a.data_ptr()
    if tscale_w is not None:
        d.tscale_w = tscale_w.data_ptr()
    if clock_probe is not None:
        d.clock_probe = clock_probe.data_ptr()
    if bias_scale is not None:
        d.bias_scale = bias_scale.data_ptr()
    if out is None and out_shape is not None:
        out = torch.empty(out_shape, dtype=torch.bfloat16, device=A.device)
    if nws > 0:
        if workspace is None or workspace.numel() < nws:
            workspace = torch.empty((nws,), dtype=torch.uint8, device=A.device)
        wsp, wsn = workspace.data_ptr(), workspace.numel()
    else:
        wsp, wsn = None, 0
    _check(lib.gemm_scaled(_ptr(out), A.data_ptr(), _ptr(sa), W.data_ptr(), _ptr(sw), _ptr(residual), epi,
                           ctypes.byref(d), wsp, wsn, _stream(A)), "gemm_scaled")
    return segs if segs is not None else out


_GEMM_CACHE: dict = {}
_GEMM_CACHE_MAX = 256


def _sig(t):
    """What the argument checks read of a tensor: shape, strides, dtype,
    device and the pointer's alignment (TypeError for a non-tensor)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError
    return (t.shape, t.stride(), t.dtype, t.device, t.data_ptr() & 15)


def _prepare(A, sa, W, sw, fmt, epilogue, out, residual, tscale_a, tscale_w, scale_layout, bias_scale,
             a_kmajor, w_kmajor):
    """Checks a gemm_scaled call without an output split and returns its
    descriptor with the pointer fields cleared (as bytes), the epilogue code,
    the shape of the output to allocate when none is given, and the
    workspace bytes the library asks for."""
    check_operands(A, sa, W, sw, fmt, epilogue, out, residual, tscale_a, tscale_w, scale_layout, bias_scale,
                   None, a_kmajor, w_kmajor)
    _need(A.is_cuda, "operands must be CUDA tensors")
    d, epi, batched = make_desc(A, W, fmt, epilogue, out, residual, tscale_a, tscale_w, a_kmajor, w_kmajor)
    d.scale_layout = _LAYOUT.get(scale_layout, scale_layout)
    if bias_scale is not None:
        d.bias_scale = bias_scale.data_ptr()
    nws = lib.gemm_scaled_workspace_bytes(ctypes.byref(d), epi)
    d.tscale_a = d.tscale_w = d.bias_scale = None
    n_out = d.N // 2 if epi == EPI_SWIGLU else d.N
    out_shape = (d.batch, d.M, n_out) if batched else (d.M, n_out)
    return bytes(d), epi, out_shape, nws


def gemm_workspace(A, W, fmt="e4m3_row", epilogue="store", out=None, residual=None, a_kmajor=False,
                   w_kmajor=False):
    """A device workspace large enough for gemm_scaled on these operands, or
    None when the plan needs none."""
    d, epi, _ = make_desc(A, W, fmt, epilogue, out, residual, a_kmajor=a_kmajor, w_kmajor=w_kmajor)
    nws = lib.gemm_scaled_workspace_bytes(ctypes.byref(d), epi)
    return torch.empty((nws,), dtype=torch.uint8, device=A.device) if nws > 0 else None


def gemm_plan(M, N, K, fmt="e4m3_row", epilogue="store", batch=1, units=256) -> dict:
    fmt = _FMT.get(fmt, fmt)
    epi = _EPI.get(epilogue, epilogue)
    d = _desc(fmt, M, N, K)
    d.batch = batch
    if batch > 1:
        d.stride_a, d.stride_w = M * d.lda, N * d.ldw
    p = Plan()
    _check(lib.spg_gemm_plan(ctypes.byref(d), epi, units, ctypes.byref(p)), "spg_gemm_plan")
    return {f: getattr(p, f) for f, _ in Plan._fields_}


def route_cost(bm, bn, per_unit, factor, M, N, batch, units) -> float:
    c = RouteCandidate(bm, bn, per_unit, factor)
    return lib.spg_route_cost(ctypes.byref(c), M, N, batch, units)


def route_select(cands, M, N, batch, units) -> int:
    arr = (RouteCandidate * len(cands))(*[RouteCandidate(*c) for c in cands])
    return lib.spg_route_select(arr, len(cands), M, N, batch, units)


# ---- measurement probes (not steps of the method) ------------------------
PROBE_MFMA_FLOPS = {0: 131072, 1: 32768}     # per MFMA: E4M3 32x32x64, f16 32x32x16


def probe_mfma(kind: int, iters: int, workgroups: int, device="cuda"):
    """Enqueue the MFMA-only probe on the current stream; returns (sink,
    clocks) device tensors (see spg_probe_mfma) and the flops it performs."""
    sink = torch.empty((workgroups * 256,), dtype=torch.float32, device=device)
    clocks = torch.zeros((4,), dtype=torch.int64, device=device)
    _check(lib.spg_probe_mfma(kind, iters, workgroups, _ptr(sink), _ptr(clocks), _stream(sink)), "spg_probe_mfma")
    return sink, clocks, workgroups * 4 * iters * 4 * PROBE_MFMA_FLOPS[kind]


def probe_fp4_rounding(device="cuda") -> dict:
    """Compare the E2M1 conversion instruction with the library's encoder on
    every non-NaN binary32 input (see spg_probe_fp4_rounding)."""
    res = torch.empty((34,), dtype=torch.int32, device=device)
    _check(lib.spg_probe_fp4_rounding(_ptr(res), _stream(res)), "spg_probe_fp4_rounding")
    h = res.cpu().numpy().view("uint32")
    n = int(min(h[1], 16))
    return {"differences": int(h[0]), "examples": [(int(h[2 + 2 * k]), int(h[3 + 2 * k])) for k in range(n)]}


def probe_read(buf: torch.Tensor, workgroups: int):
    """Enqueue the HBM read probe over the bytes of contiguous `buf` on the
    current stream; returns the sink (one XOR-folded word per thread)."""
    _need(buf.is_contiguous(), "probe_read: buf must be contiguous")
    sink = torch.empty((workgroups * 256,), dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(lib.spg_probe_read(_ptr(buf), nbytes, workgroups, _ptr(sink), _stream(buf)), "spg_probe_read")
    return sink

