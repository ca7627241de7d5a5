"""Host-side tests of the C ABI (no GPU needed, nothing is launched).

* The library loads and exports every function include/spg.h declares.
* Every validation error path returns its status before any launch (the
  data pointers passed here are never dereferenced).
* The tile / split-K plan for the workloads.
* The route cost model, parameterized with the RTX 5090 geometry of ninfer
  PR #167, reproduces every decision that page prints.
"""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "spg.h")


@pytest.fixture(scope="module")
def spg():
    lib = os.path.join(ROOT, "scaled_precision_gemm_amd", "libspg.so")
    if not os.path.exists(lib):
        subprocess.run(["python", os.path.join(ROOT, "scaled_precision_gemm_amd", "build.py")], check=True)
    import scaled_precision_gemm_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{}()]*(?:\([^()]*\)[^;{}()]*)*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("sizeof",)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("quantize_rowwise", "quantize_block16", "quantize_tensor", "gemm_scaled",
              "gemm_scaled_workspace_bytes", "spg_gemm_plan", "spg_route_select"):
        assert n in names


def test_library_exports_every_declared_function(spg):
    names = declared_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", spg.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(line.split()[-1] for line in out.stdout.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert set(names) <= set(spg.SIGNATURES)


def test_status_strings(spg):
    assert spg.lib.spg_status_string(0) == b"success"
    assert spg.lib.spg_status_string(3) == b"workspace missing or too small"
    assert spg.lib.spg_status_string(99) == b"unknown status"


# ---------------------------------------------------------------------------
# validation (fake, aligned, never-dereferenced pointers)
# ---------------------------------------------------------------------------
P = ctypes.c_void_p
FAKE = P(0x100000)
FAKE2 = P(0x40000000000)     # far from FAKE: no overlap with any output here
MIS = P(0x100001)
EINVAL, EUNSUP, EWS = 1, 2, 3


def desc(spg, M, N, K, fmt=0):
    d = spg.GemmDesc()
    spg.lib.spg_gemm_desc_init(ctypes.byref(d), M, N, K, fmt)
    return d


def call_gemm(spg, d, epi=0, out=FAKE, A=FAKE, sa=FAKE, W=FAKE, sw=FAKE, res=None, ws=None, nws=0):
    return spg.lib.gemm_scaled(out, A, sa, W, sw, res, epi, ctypes.byref(d) if d is not None else None,
                               ws, nws, None)


def test_desc_init_defaults(spg):
    d = desc(spg, 10, 20, 64, 0)
    assert (d.M, d.N, d.K, d.batch, d.lda, d.ldw, d.ldo, d.ldr) == (10, 20, 64, 1, 64, 64, 20, 20)
    assert d.stride_a == d.stride_w == d.stride_o == d.stride_r == 0
    assert not d.tscale_a and not d.tscale_w
    d4 = desc(spg, 10, 20, 64, 2)
    assert d4.lda == d4.ldw == 32


@pytest.mark.parametrize("case", [
    "null_desc", "bad_format", "bad_epilogue", "k_not_16", "nvfp4_k_not_32", "lda_short", "lda_unaligned",
    "ldo_short", "swiglu_odd_n", "add_without_residual", "store_with_residual", "null_a", "misaligned_a",
    "negative_m", "zero_batch", "nvfp4_no_tscale", "negative_stride", "ldr_short", "bias_row_in_place",
    "in_place_other_ldr", "in_place_other_batch_stride", "residual_overlaps_out", "bias_row_inside_out",
    "output_batches_overlap", "output_broadcast", "bias_scale_with_store", "bias_scale_with_matrix_residual",
    "bias_scale_misaligned", "bias_scale_inside_out", "e4m3_bias_row_inside_out",
])
def test_gemm_validation_errors(spg, case):
    d = desc(spg, 64, 64, 64, 0)
    kw = {}
    epi = 0
    if case == "null_desc":
        d = None
    elif case == "bad_format":
        d.format = 7
    elif case == "bad_epilogue":
        epi = 5
    elif case == "k_not_16":
        d = desc(spg, 64, 64, 72, 0)
    elif case == "nvfp4_k_not_32":
        d = desc(spg, 64, 64, 48, 2)
    elif case == "lda_short":
        d.lda = 32
    elif case == "lda_unaligned":
        d.lda = 72
    elif case == "ldo_short":
        d.ldo = 32
    elif case == "swiglu_odd_n":
        d = desc(spg, 64, 63, 64, 0)
        epi = 2
    elif case == "add_without_residual":
        epi = 1
    elif case == "store_with_residual":
        kw["res"] = FAKE2
    elif case == "null_a":
        kw["A"] = None
    elif case == "misaligned_a":
        kw["A"] = MIS
    elif case == "negative_m":
        d.M = -1
    elif case == "zero_batch":
        d.batch = 0
    elif case == "nvfp4_no_tscale":
        d = desc(spg, 64, 64, 64, 2)
    elif case == "negative_stride":
        d.stride_a = -16
    elif case == "ldr_short":
        epi, d.ldr, kw["res"] = 1, 32, FAKE2
    elif case == "bias_row_in_place":
        # ldr == 0 (one bias row) with the output as that row
        epi, d.ldr, kw["res"] = 1, 0, FAKE
    elif case == "in_place_other_ldr":
        # residual == out but read with another row stride
        epi, d.ldr, d.ldo, kw["res"] = 1, 64, 128, FAKE
    elif case == "in_place_other_batch_stride":
        d.batch, d.stride_a, d.stride_o, d.stride_r = 2, 64 * 64, 64 * 64, 64 * 128
        epi, kw["res"] = 1, FAKE
    elif case == "residual_overlaps_out":
        # residual starts one row inside the output
        epi, kw["res"] = 1, P(FAKE.value + 2 * 64)
    elif case == "bias_row_inside_out":
        epi, d.ldr, kw["res"] = 1, 0, P(FAKE.value + 2 * 64 * 10)
    elif case == "output_batches_overlap":
        d.batch, d.stride_a, d.stride_o = 2, 64 * 64, 64 * 63
    elif case == "output_broadcast":
        d.batch, d.stride_a, d.stride_o = 2, 64 * 64, 0
    elif case == "bias_scale_with_store":
        d.bias_scale = FAKE2.value
    elif case == "bias_scale_with_matrix_residual":
        # an E4M3 bias is one row (ldr == 0), never a residual matrix
        epi, kw["res"], d.bias_scale = 1, FAKE2, FAKE2.value + 4096
    elif case == "bias_scale_misaligned":
        epi, d.ldr, kw["res"], d.bias_scale = 1, 0, FAKE2, FAKE2.value + 4098
    elif case == "bias_scale_inside_out":
        epi, d.ldr, kw["res"], d.bias_scale = 1, 0, FAKE2, FAKE.value + 256
    elif case == "e4m3_bias_row_inside_out":
        epi, d.ldr, kw["res"], d.bias_scale = 1, 0, P(FAKE.value + 2 * 64 * 63 + 1), FAKE2.value
    assert call_gemm(spg, d, epi, **kw) == EINVAL


def test_gemm_in_place_and_disjoint_residuals_pass_validation(spg):
    # exactly aliased (same pointer, row and batch stride) and disjoint
    # residuals get past validation: with no device the call then fails at
    # the launch (SPG_EHIP) or, given a GPU, runs; never SPG_EINVAL
    d = desc(spg, 64, 64, 64, 0)
    assert call_gemm(spg, d, 1, res=FAKE) != EINVAL
    assert call_gemm(spg, d, 1, res=P(FAKE.value + 2 * 64 * 64)) != EINVAL
    d.batch, d.stride_a, d.stride_o, d.stride_r = 2, 64 * 64, 64 * 64, 64 * 64
    assert call_gemm(spg, d, 1, res=FAKE) != EINVAL


def test_gemm_bias_row_is_a_valid_residual(spg):
    # ldr == 0 passes validation (the plan and workspace queries accept it)
    d = desc(spg, 64, 64, 64, 0)
    d.ldr = 0
    p = spg.Plan()
    assert spg.lib.spg_gemm_plan(ctypes.byref(d), 1, 256, ctypes.byref(p)) == 0
    assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 1) == 0


def test_gemm_e4m3_bias_row_passes_validation(spg):
    # E4M3 bias codes are single bytes: any address outside the output, even
    # an odd one, with a 4-byte aligned scale outside the output, gets past
    # validation (SPG_EHIP without a device, never SPG_EINVAL); the byte just
    # past the output's last element is outside it
    d = desc(spg, 64, 64, 64, 0)
    d.ldr, d.bias_scale = 0, FAKE2.value
    assert call_gemm(spg, d, 1, res=P(FAKE2.value + 4097)) != EINVAL
    assert call_gemm(spg, d, 1, res=P(FAKE.value + 2 * 64 * 64)) != EINVAL
    d.bias_scale = FAKE.value + 2 * 64 * 64
    assert call_gemm(spg, d, 1, res=FAKE2) != EINVAL
    p = spg.Plan()
    assert spg.lib.spg_gemm_plan(ctypes.byref(d), 1, 256, ctypes.byref(p)) == 0


def out_split(spg, widths, ptrs, ldos, strides=None):
    sp = spg.OutSplit()
    sp.count = len(widths)
    end = 0
    for i, w in enumerate(widths):
        end += w
        sp.col_end[i] = end
        sp.out[i] = ptrs[i]
        sp.ldo[i] = ldos[i]
        sp.stride_o[i] = strides[i] if strides else 0
    return sp


SEG = [0x10000000, 0x20000000, 0x30000000]       # far apart, 16-byte aligned


@pytest.mark.parametrize("case", [
    "count_zero", "count_nine", "out_also_given", "boundary_not_64", "last_short", "ends_not_increasing",
    "segment_misaligned", "ldo_short", "ldo_not_8", "segments_overlap", "residual_in_segment",
    "batch_stride_short", "null_segment",
])
def test_gemm_out_split_validation(spg, case):
    # N = 320 outputs as 128 | 128 | 64 by default
    d = desc(spg, 64, 320, 64, 0)
    widths, ptrs, ldos, strides = [128, 128, 64], list(SEG), [128, 128, 64], None
    epi, kw = 0, {"out": None}
    if case == "count_zero":
        widths = []
    elif case == "count_nine":
        widths, ptrs, ldos = [64] * 5, SEG + [0x40000000, 0x50000000], [64] * 5
    elif case == "out_also_given":
        kw["out"] = FAKE
    elif case == "boundary_not_64":
        widths = [96, 160, 64]
    elif case == "last_short":
        widths = [128, 128, 32]
    elif case == "ends_not_increasing":
        widths = [128, 0, 192]
    elif case == "segment_misaligned":
        ptrs[1] += 8
    elif case == "ldo_short":
        ldos[0] = 120
    elif case == "ldo_not_8":
        ldos[2] = 68
    elif case == "segments_overlap":
        ptrs[1] = SEG[0] + 2 * 64 * 128 - 16      # inside segment 0's last row
    elif case == "residual_in_segment":
        epi, kw["res"] = 1, P(SEG[2] + 64)
    elif case == "batch_stride_short":
        d.batch, d.stride_a = 2, 64 * 64
        strides = [64 * 128, 63 * 128, 64 * 64]
    elif case == "null_segment":
        ptrs[2] = 0
    sp = out_split(spg, widths, ptrs, ldos, strides)
    if case == "count_nine":
        sp.count = 9
    d.out_split = ctypes.pointer(sp)
    assert call_gemm(spg, d, epi, **kw) == EINVAL


def test_gemm_out_split_passes_validation(spg):
    # a valid split (also with a residual elsewhere, and batched) gets past
    # validation: SPG_EHIP without a device, never SPG_EINVAL
    d = desc(spg, 64, 320, 64, 0)
    sp = out_split(spg, [128, 128, 64], SEG, [128, 136, 64])
    d.out_split = ctypes.pointer(sp)
    assert call_gemm(spg, d, 0, out=None) != EINVAL
    assert call_gemm(spg, d, 1, out=None, res=FAKE2) != EINVAL
    d2 = desc(spg, 64, 640, 64, 0)
    sp2 = out_split(spg, [320], [SEG[0]], [320])
    d2.out_split = ctypes.pointer(sp2)
    assert call_gemm(spg, d2, 2, out=None) != EINVAL       # SwiGLU: 320 outputs
    d.batch, d.stride_a = 2, 64 * 64
    sp3 = out_split(spg, [128, 128, 64], SEG, [128, 128, 64], [64 * 128, 64 * 128, 64 * 64])
    d.out_split = ctypes.pointer(sp3)
    assert call_gemm(spg, d, 0, out=None) != EINVAL


def test_gemm_kmajor_layout_validation(spg):
    # K-major operands: stored row strides are checked against M / N, the
    # flags against their range, NVFP4 takes none
    d = desc(spg, 32, 48, 64, 0)
    d.layout = 4
    assert call_gemm(spg, d) == EINVAL
    d = desc(spg, 32, 48, 64, 0)
    d.layout, d.lda = 1, 16                     # A stored [64, 32]: lda >= 32
    assert call_gemm(spg, d) == EINVAL
    d.lda = 32                                  # (NT would need lda >= K = 64)
    assert call_gemm(spg, d) != EINVAL
    d.layout, d.lda, d.ldw = 2, 64, 32          # W stored [64, 48]: ldw >= 48
    assert call_gemm(spg, d) == EINVAL
    d.ldw = 48
    assert call_gemm(spg, d) != EINVAL
    d4 = desc(spg, 64, 64, 64, 2)
    d4.layout = 2
    assert call_gemm(spg, d4) == EUNSUP


def test_gemm_kmajor_workspace_holds_the_transposed_copies(spg):
    # one 256-byte aligned [M, K] (and [N, K]) copy per batch entry of each
    # K-major operand, ahead of any K-split partials
    d = desc(spg, 300, 520, 1040, 1)
    base = spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 0)
    for layout, extra in ((1, 300 * 1040), (2, 520 * 1040), (3, 300 * 1040 + 520 * 1040)):
        d.layout = layout
        al = lambda b: (b + 255) // 256 * 256
        want = al(300 * 1040) * (layout & 1) + al(520 * 1040) * ((layout >> 1) & 1)
        assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 0) == base + want
    # batched with a broadcast W: A copies per entry, one W copy
    d = desc(spg, 64, 64, 128, 1)
    d.batch, d.stride_a, d.layout, d.lda = 3, 128 * 64, 3, 64
    d.ldw = 64
    d.stride_o = 64 * 64
    assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 0) == 3 * 64 * 128 + 64 * 128


def test_gemm_nvfp4_batch_unsupported(spg):
    d = desc(spg, 64, 64, 64, 2)
    d.batch = 2
    assert call_gemm(spg, d) == EUNSUP


def test_gemm_stride_limits_unsupported(spg):
    d = desc(spg, 64, 64, 64, 0)
    d.lda = 1 << 24
    assert call_gemm(spg, d) == EUNSUP
    d = desc(spg, 64, 64, 64, 0)
    d.ldo = 1 << 26
    assert call_gemm(spg, d) == EUNSUP
    d = desc(spg, 64, 64, 64, 0)
    d.ldr = 1 << 26
    assert call_gemm(spg, d, 1, res=FAKE2) == EUNSUP


def test_gemm_workspace_too_small(spg):
    # T=1024 down-projection: 80 output tiles on 256 CUs -> a K split
    d = desc(spg, 1024, 5120, 17408, 0)
    assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 1) > 0
    assert call_gemm(spg, d, 1, res=FAKE2) == EWS
    assert call_gemm(spg, d, 1, res=FAKE2, ws=FAKE, nws=1024) == EWS


def test_gemm_empty_is_noop(spg):
    assert call_gemm(spg, desc(spg, 0, 64, 64)) == 0
    assert call_gemm(spg, desc(spg, 64, 0, 64)) == 0


def test_quantizer_validation_errors(spg):
    L = spg.lib
    assert L.quantize_rowwise(FAKE, 4, 8, 8, FAKE, 16, FAKE, None) == EINVAL          # K % 16
    assert L.quantize_rowwise(FAKE, 4, 32, 16, FAKE, 32, FAKE, None) == EINVAL        # ldx < K
    assert L.quantize_rowwise(FAKE, 4, 32, 32, None, 32, FAKE, None) == EINVAL        # null q
    assert L.quantize_rowwise(MIS, 4, 32, 32, FAKE, 32, FAKE, None) == EINVAL         # misaligned
    assert L.quantize_rowwise(FAKE, 4, 32, 32, FAKE, 40, FAKE, None) == EINVAL        # ldq % 16
    assert L.quantize_rowwise(FAKE, 4, 0, 0, FAKE, 0, FAKE, None) == EINVAL           # empty rows
    assert L.quantize_rowwise(FAKE, 0, 32, 32, FAKE, 32, FAKE, None) == 0             # no rows: no-op
    nws = L.quantize_tensor_workspace_bytes(2, 64, 64)
    assert nws >= 8
    assert L.quantize_tensor(FAKE, 2, 64, 64, 4096, FAKE, FAKE, None, 0, None) == EWS
    assert L.quantize_tensor(FAKE, 2, 64, 64, 4096, FAKE, FAKE, FAKE, nws - 4, None) == EWS
    assert L.quantize_tensor(FAKE, 2, 64, 64, 4000, FAKE, FAKE, FAKE, nws, None) == EINVAL  # bstride < rows*K
    assert L.quantize_tensor(FAKE, 0, 64, 64, 4096, FAKE, FAKE, FAKE, nws, None) == EINVAL
    nb = L.quantize_block16_workspace_bytes(64, 64)
    assert nb >= 4 * (4 + 1)                     # election words + at least one partial
    ROW, BLK = 0, 1
    assert L.quantize_block16(FAKE, 64, 48, FAKE, FAKE, FAKE, ROW, FAKE, nb, None) == EINVAL     # K % 32
    assert L.quantize_block16(FAKE, 64, 64, FAKE, FAKE, FAKE, ROW, None, 0, None) == EWS
    assert L.quantize_block16(FAKE, 64, 64, None, FAKE, FAKE, ROW, FAKE, nb, None) == EINVAL
    assert L.quantize_block16(FAKE, 64, 64, FAKE, FAKE, FAKE, 2, FAKE, nb, None) == EINVAL       # bad layout
    assert L.quantize_block16(FAKE, 64, 64, FAKE, FAKE, FAKE, 0x200, FAKE, nb, None) == EINVAL   # unknown flag
    assert L.quantize_block16(FAKE, 64, 224, FAKE, FAKE, FAKE, BLK, FAKE, nb, None) == EINVAL    # blocked: K % 256
    assert L.quantize_block16_noalloc(FAKE, 64, 48, FAKE, FAKE, FAKE, ROW, None) == EINVAL
    assert L.quantize_block16_noalloc(FAKE, 64, 224, FAKE, FAKE, FAKE, BLK, None) == EINVAL
    assert L.quantize_block16_noalloc(MIS, 64, 64, FAKE, FAKE, FAKE, ROW, None) == EINVAL


def test_gemm_scale_layout_validation(spg):
    # blocked NVFP4 planes need K % 256 == 0; the field must be zero for FP8
    d = desc(spg, 64, 64, 224, 2)
    d.scale_layout = 1
    assert call_gemm(spg, d) == EINVAL
    d = desc(spg, 64, 64, 256, 2)
    d.scale_layout = 3
    assert call_gemm(spg, d) == EINVAL
    d = desc(spg, 64, 64, 64, 0)
    d.scale_layout = 1
    assert call_gemm(spg, d) == EINVAL
    d = desc(spg, 64, 64, 256, 2)
    d.scale_layout = 1
    p = spg.Plan()
    assert spg.lib.spg_gemm_plan(ctypes.byref(d), 0, 256, ctypes.byref(p)) == 0


# ---------------------------------------------------------------------------
# plans for the workloads (256 compute units)
# ---------------------------------------------------------------------------

def test_plans_for_the_workloads(spg):
    # 80 tiles on 256 units: a 3-way K split, one workgroup per (tile, slice)
    p = spg.gemm_plan(1024, 5120, 17408, "e4m3_row", "add")
    assert (p["bm"], p["bn"], p["bk"], p["tiles"], p["split_k"], p["workgroups"]) == (256, 256, 128, 80, 3, 240)
    # unsplit FP8 products with two or more K stages: one persistent workgroup per unit
    p = spg.gemm_plan(4096, 34816, 5120, "e4m3_row", "swiglu")
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (16 * 136, 1, 256)
    p = spg.gemm_plan(4096, 34816, 5120, "e4m3_row", "swiglu", units=304)
    assert p["workgroups"] == 304
    # at most 32 tokens: the decode-width kernel, one workgroup per 32 output
    # columns (SwiGLU: 16 columns, 16 gate + 16 up rows), no K split, no
    # workspace
    p = spg.gemm_plan(16, 34816, 5120, "e4m3_row", "swiglu")
    assert (p["kernel"], p["bm"], p["bn"], p["tiles"], p["split_k"], p["workgroups"]) == (3, 16, 16, 1088, 1, 1088)
    p = spg.gemm_plan(16, 5120, 17408, "e4m3_row", "add")
    assert (p["kernel"], p["bn"], p["tiles"], p["split_k"], p["workgroups"]) == (3, 32, 160, 1, 160)
    p = spg.gemm_plan(32, 5120, 6144, "nvfp4", "add")
    assert (p["kernel"], p["bm"], p["bk"], p["workgroups"]) == (3, 32, 256, 160)
    # NVFP4 with K % 64 != 0 (scale rows of whole 4-byte words only): tiled
    assert spg.gemm_plan(16, 5120, 6176, "nvfp4", "add")["kernel"] == 1
    # fewer than 32 column blocks: the tiled route (unsplit: 128-row tiles)
    assert spg.gemm_plan(16, 496, 512, "e4m3_row", "store")["kernel"] == 2
    assert spg.gemm_plan(1, 512, 512, "e4m3_tensor", "store")["kernel"] == 3
    # 33 to 64 tokens: the weight-streaming cost model (waves * (slice + 1024))
    # picks 3 slices for the SwiGLU (408 workgroups, 1.6 waves beat 2.7 at
    # 5 slices) and keeps 8 for the down-projection (one wave of 160)
    p = spg.gemm_plan(48, 34816, 5120, "e4m3_row", "swiglu")
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (136, 3, 408)
    p = spg.gemm_plan(48, 5120, 17408, "e4m3_row", "add")
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (20, 8, 160)
    # NVFP4 at 48 tokens (fast path, K % 256 == 0) takes the weight-streaming
    # model too; with K % 256 != 0 (general path) the wave-quantised one
    p = spg.gemm_plan(48, 34816, 5120, "nvfp4", "swiglu")
    assert (p["split_k"], p["workgroups"]) == (3, 408)
    p = spg.gemm_plan(48, 34816, 5152, "nvfp4", "swiglu")
    assert p["split_k"] == 5
    # no K slice is ever empty
    for K in (8448, 9472, 12544, 14080):
        for fmt in ("nvfp4", "e4m3_row"):
            p = spg.gemm_plan(48, 5120, K, fmt, "add")
            s, bk = p["split_k"], p["bk"]
            chunk = -(-(-(-K // s)) // bk) * bk
            assert (s - 1) * chunk < K, (K, fmt, s)
    # 128 tokens, one tile: one 128-row half tile (the lower half of a
    # 256-row tile would hold no rows)
    p = spg.gemm_plan(128, 256, 512, "e4m3_row", "store")
    assert (p["tiles"], p["split_k"], p["workgroups"], p["bm"], p["kernel"]) == (1, 1, 1, 128, 2)
    p = spg.gemm_plan(512, 512, 512, "e4m3_tensor", "store", batch=64)
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (256, 1, 256)
    p = spg.gemm_plan(8192, 8192, 8192, "e4m3_tensor", "store")
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (1024, 1, 256)
    # a single K stage runs one workgroup per tile
    p = spg.gemm_plan(4096, 4096, 128, "e4m3_tensor", "store")
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (256, 1, 256)
    p = spg.gemm_plan(8192, 4096, 128, "e4m3_tensor", "store")
    assert (p["tiles"], p["split_k"], p["workgroups"]) == (512, 1, 512)
    # NVFP4: 320 tiles = one round of 256 + 64 more; the 64 run split 4 ways
    # along K in a second launch (tail split), the first launch takes 256
    p = spg.gemm_plan(4096, 5120, 6144, "nvfp4", "add")
    assert (p["tiles"], p["split_k"], p["bk"], p["workgroups"]) == (320, 1, 256, 256)
    assert (p["tail_tiles"], p["tail_split"]) == (64, 4)
    # FP8 at T=4096 SwiGLU: 8.5 rounds; a K split of the last half round of
    # 70 us tiles does not pay for the partial-tile traffic, half-height
    # tiles (no partials) do: 8 whole rounds, then 256 halves of 128 tiles
    p = spg.gemm_plan(4096, 34816, 5120, "e4m3_row", "swiglu")
    assert (p["workgroups"], p["tail_tiles"], p["tail_split"], p["tail_bm"]) == (256, 128, 1, 128)
    # 16 tiles left, K 2048: half-height tiles (a K split of 2048 is too short)
    p = spg.gemm_plan(4096, 4352, 2048, "e4m3_row", "store")
    assert (p["tiles"], p["tail_tiles"], p["tail_split"], p["tail_bm"]) == (272, 16, 1, 128)
    # K 1024: the tail's launch outweighs a short round; 128-row tiles over
    # the whole product (3 rounds at 0.62) are priced below it
    p = spg.gemm_plan(4096, 4352, 1024, "e4m3_row", "store")
    assert (p["kernel"], p["tiles"], p["workgroups"], p["tail_tiles"]) == (2, 544, 544, 0)
    # more than half a round left: no half-height tail (it would take 2 rounds)
    p = spg.gemm_plan(4096, 4096 + 12 * 256, 5120, "e4m3_row", "store")
    assert p["tiles"] == 16 * 28 and p["tail_bm"] == 256
    # NVFP4 has no half-height kernel
    assert spg.gemm_plan(4096, 5120, 6144, "nvfp4", "add")["tail_bm"] == 256
    # long K: worth it for FP8 too (K / 8 still >= 1024)
    p = spg.gemm_plan(4096, 4352, 16384, "e4m3_row", "store")
    assert (p["tiles"], p["workgroups"], p["tail_tiles"], p["tail_split"], p["tail_bm"]) == (272, 256, 16, 8, 256)
    # whole rounds: no tail
    p = spg.gemm_plan(8192, 8192, 8192, "e4m3_tensor", "store")
    assert (p["tail_tiles"], p["tail_split"]) == (0, 1)
    p = spg.gemm_plan(4096, 5120, 6176, "nvfp4", "add")   # K not a multiple of 256: general path
    assert (p["tiles"], p["bk"]) == (320, 64)


def test_workspace_covers_the_tail_split(spg):
    d = desc(spg, 4096, 5120, 6144, 2)
    assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 1) == 64 * 4 * 256 * 256 * 4
    d = desc(spg, 4096, 34816, 5120, 0)
    assert spg.lib.gemm_scaled_workspace_bytes(ctypes.byref(d), 2) == 0


# ---------------------------------------------------------------------------
# the route model against ninfer PR #167's printed decisions
# ---------------------------------------------------------------------------

def load_decisions():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "p1_fp8_route_decisions.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "table":
            N, K, site, T, ratio = int(f[1]), int(f[2]), f[3], int(f[4]), float(f[5])
            rows.append(("table", N, K, T, ratio < 1.0, (N, K, T) == (5120, 6144, 8192)))
        else:
            rows.append(("sweep", int(f[1]), int(f[2]), int(f[3]), f[4] == "taken", False))
    return rows


# RTX 5090 geometry from the page's table: the TMA route runs 256-token x
# 128-row tiles one CTA per SM; the cp.async route 64 x 128 tiles two per SM;
# one empirical factor (0.936) on the TMA route's cost; 170 SMs.
TMA = (256, 128, 1, 0.936)
CPA = (64, 128, 2, 1.0)


@pytest.mark.parametrize("row", load_decisions(), ids=lambda r: f"{r[0]}-{r[1]}x{r[2]}-T{r[3]}")
def test_route_model_reproduces_printed_decisions(spg, row):
    kind, N, K, T, taken, ceiling = row
    pick = spg.route_select([TMA, CPA], T, N, 1, 170)
    if ceiling:
        # declined by the page's per-geometry ceiling, which the cost model
        # cannot express: the model alone takes it
        assert not taken and pick == 0
    else:
        assert (pick == 0) == taken


def test_route_cost_is_waves_times_work_per_sm(spg):
    # 14336 rows, T=1024: 4 x 112 = 448 TMA tiles -> 3 waves of 170
    assert spg.route_cost(256, 128, 1, 1.0, 1024, 14336, 1, 170) == 3 * 256 * 128
    # 16 x 112 = 1792 cp.async tiles over 340 slots -> 6 waves of 2 x 64 x 128
    assert spg.route_cost(64, 128, 2, 1.0, 1024, 14336, 1, 170) == 6 * 2 * 64 * 128


def test_probe_validation_errors(spg):
    # every case is rejected before anything is enqueued (no GPU needed)
    P = ctypes.c_void_p
    buf = P(0x10000)
    assert spg.lib.spg_probe_mfma(2, 10, 1, buf, buf, None) == 1          # unknown kind
    assert spg.lib.spg_probe_mfma(0, 0, 1, buf, buf, None) == 1           # no iterations
    assert spg.lib.spg_probe_mfma(1, 10, 0, buf, buf, None) == 1          # no workgroups
    assert spg.lib.spg_probe_mfma(0, 10, 1, None, buf, None) == 1         # null sink
    assert spg.lib.spg_probe_mfma(0, 10, 1, buf, P(0x10004), None) == 1  # clocks not 8-byte aligned
    assert spg.lib.spg_probe_read(None, 1024, 1, buf, None) == 1
    assert spg.lib.spg_probe_read(buf, 1000, 1, buf, None) == 1          # not a multiple of 16
    assert spg.lib.spg_probe_read(P(0x10008), 1024, 1, buf, None) == 1   # source not 16-byte aligned
    assert spg.lib.spg_probe_read(buf, 1024, 0, buf, None) == 1
    assert spg.lib.spg_probe_fp4_rounding(None, None) == 1               # null result
    assert spg.lib.spg_probe_fp4_rounding(P(0x10002), None) == 1         # not 4-byte aligned


# ---------------------------------------------------------------------------
# the MI355X plan: tile geometry (ninfer PR #167's route model, recalibrated
# for 256 compute units: 256 x 256 factor 1, 128 x 256 factor 1.24), split-K,
# tails; the decisions for the benchmark workloads and the cases where the
# 128-row geometry is taken
# ---------------------------------------------------------------------------
MI355X_PLANS = [
    # (M, N, K, fmt, epi, batch) -> (kernel, bm, split_k, tail_tiles, tail_split, tail_bm)
    ((128, 256, 512, "e4m3_row", "store", 1), (2, 128, 1, 0, 1, 256)),       # 128-row tiles where they measured faster
    ((96, 34816, 5120, "e4m3_row", "swiglu", 1), (2, 128, 1, 0, 1, 256)),
    ((257, 300, 160, "e4m3_row", "store", 1), (2, 128, 1, 0, 1, 256)),
    ((288, 21760, 4096, "e4m3_row", "store", 1), (2, 128, 1, 0, 1, 256)),
    ((352, 21760, 4096, "e4m3_row", "add", 1), (2, 128, 1, 0, 1, 256)),
    ((384, 21760, 8192, "e4m3_row", "store", 1), (2, 128, 1, 0, 1, 256)),
    ((384, 43008, 4096, "e4m3_row", "store", 1), (2, 128, 1, 0, 1, 256)),
    ((300, 43520, 4096, "e4m3_row", "swiglu", 1), (2, 128, 1, 0, 1, 256)),
    ((640, 26624, 4096, "e4m3_row", "store", 1), (0, 256, 1, 56, 1, 128)),   # 256-row tiles where they measured faster
    ((200, 40000, 4096, "e4m3_row", "store", 1), (0, 256, 1, 0, 1, 256)),
    ((2048, 8192, 4096, "e4m3_row", "store", 1), (0, 256, 1, 0, 1, 256)),
    ((160, 65536, 2048, "e4m3_row", "store", 1), (0, 256, 1, 0, 1, 256)),
    ((1536, 16384, 4096, "e4m3_row", "store", 1), (0, 256, 1, 128, 1, 128)),
    ((128, 5120, 4096, "e4m3_row", "add", 1), (0, 256, 4, 0, 1, 256)),       # split along K: no geometry choice
    ((1024, 5120, 17408, "e4m3_row", "add", 1), (0, 256, 3, 0, 1, 256)),    # 80 tiles: K split 3
    ((4096, 34816, 5120, "e4m3_row", "swiglu", 1), (0, 256, 1, 128, 1, 128)),  # 8.5 rounds: half-height tail
    ((4096, 5120, 6144, "e4m3_row", "add", 1), (0, 256, 1, 64, 1, 128)),
    ((4096, 7168, 5120, "e4m3_row", "store", 1), (0, 256, 1, 0, 1, 256)),
    ((4096, 12288, 2048, "e4m3_row", "store", 1), (0, 256, 1, 0, 1, 256)),
    ((4096, 5120, 6144, "nvfp4", "add", 1), (1, 256, 1, 64, 4, 256)),        # NVFP4: K-split tail
    ((8192, 8192, 8192, "e4m3_tensor", "store", 1), (0, 256, 1, 0, 1, 256)),
    ((512, 512, 512, "e4m3_tensor", "store", 64), (0, 256, 1, 0, 1, 256)),
    ((48, 5120, 17408, "e4m3_row", "add", 1), (0, 256, 8, 0, 1, 256)),       # 33-64 tokens: split model
    ((48, 34816, 5120, "e4m3_row", "swiglu", 1), (0, 256, 3, 0, 1, 256)),
    ((16, 5120, 17408, "e4m3_row", "add", 1), (3, 16, 1, 0, 1, 256)),        # decode widths
    ((16, 34816, 5120, "e4m3_row", "swiglu", 1), (3, 16, 1, 0, 1, 256)),
    ((16, 5120, 6144, "nvfp4", "add", 1), (3, 16, 1, 0, 1, 256)),
    ((32, 34816, 5120, "nvfp4", "swiglu", 1), (3, 32, 1, 0, 1, 256)),
]


@pytest.mark.parametrize("case,want", MI355X_PLANS, ids=lambda v: "x".join(map(str, v[:3])) if len(v) == 6 and isinstance(v[3], str) else None)
def test_mi355x_plan_decisions(spg, case, want):
    M, N, K, fmt, epi, b = case
    p = spg.gemm_plan(M, N, K, fmt, epi, batch=b, units=256)
    assert (p["kernel"], p["bm"], p["split_k"], p["tail_tiles"], p["tail_split"], p["tail_bm"]) == want


def test_geometry_costs_follow_the_route_model(spg):
    # the planner's two candidates priced by the exported PR #167 model: a
    # round of 128-row tiles at 0.62 of a round of 256-row tiles (factor 1.24
    # on half the area), so 128-row tiles win wherever they take the same
    # number of rounds, and lose at twice the rounds
    full, half = (256, 256, 1, 1.0), (128, 256, 1, 1.24)
    assert spg.route_cost(*full, 384, 43008, 1, 256) == 2 * 256 * 256
    assert spg.route_cost(*half, 384, 43008, 1, 256) == 1.24 * 2 * 128 * 256
    assert spg.route_select([full, half], 128, 34816, 1, 256) == 1
    assert spg.route_select([full, half], 288, 21760, 1, 256) == 1
    assert spg.route_select([full, half], 2048, 8192, 1, 256) == 0
    assert spg.route_select([full, half], 4096, 34816, 1, 256) == 0
    # the planner counts the 128-row grid's tiles and launches one workgroup
    # per tile; a partial last round of 256-row tiles is priced with its tail
    for M, tiles in ((65, 168), (128, 168), (257, 504), (384, 504)):
        p = spg.gemm_plan(M, 43008, 4096, "e4m3_row", "store")
        assert (p["kernel"], p["bm"], p["workgroups"], p["tiles"]) == (2, 128, tiles, tiles)
    p = spg.gemm_plan(1024, 43008, 4096, "e4m3_row", "store")
    assert p["kernel"] == 0 and p["tiles"] == 672
    p = spg.gemm_plan(100, 4096, 512, "e4m3_tensor", "store", batch=3)
    assert (p["kernel"], p["workgroups"], p["tiles"]) == (2, 48, 48)
    p = spg.gemm_plan(1100, 7168, 512, "e4m3_row", "store")
    assert (p["kernel"], p["tiles"]) == (2, 9 * 28)
