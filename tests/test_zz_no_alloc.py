"""quantize_block16_noalloc through the C ABI against quantize_block16.

The allocation-free variant keeps its scratch (the election words of the
single-launch path, the partial maxima of the two-pass path) in a static
device array shared by every call on the GPU.  Successive calls, each
smaller and with a smaller amax than the one before, in both scale-plane
layouts: a stale word left in the array by an earlier call would change a
later call's tensor scale.  Codes, block scales and the tensor scale must
equal the workspace entry point's bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

from synthetic import bf16_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import scaled_precision_gemm_amd as m
    return m


def dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).view(torch.bfloat16).cuda()


def run(spg, x, noalloc, layout):
    R, K = x.shape
    q = torch.full((R, K // 2), 0xA5, dtype=torch.uint8, device="cuda")
    bs = torch.full(spg.block16_scale_shape(R, K, layout.split("_")[0]), 0x5A, dtype=torch.uint8, device="cuda")
    t = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())
    lay = (spg.SCALES_BLOCKED if layout.startswith("blocked") else spg.SCALES_ROW_MAJOR) | \
        (spg.QUANT_SINGLE_LAUNCH if layout.endswith("single") else 0)
    if noalloc:
        st = spg.lib.quantize_block16_noalloc(P(x), R, K, P(q), P(bs), P(t), lay, stream)
    else:
        nws = spg.lib.quantize_block16_workspace_bytes(R, K)
        ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
        st = spg.lib.quantize_block16(P(x), R, K, P(q), P(bs), P(t), lay, P(ws), ws.numel(), stream)
    assert st == 0, spg.lib.spg_status_string(st)
    torch.cuda.synchronize()
    return q.cpu().numpy(), bs.cpu().numpy(), t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("layout", ["row", "blocked", "row_single", "blocked_single"])
def test_noalloc_matches_workspace_entry_point_on_successive_calls(spg, layout):
    # three calls, each smaller and with a smaller amax than the one before;
    # with the single-launch request the first is still too large for one
    # grid (two passes: partial maxima in the scratch) and the others run as
    # one launch (counters, flag and block maxima in the scratch)
    calls = [((6144, 8448), 10.0, 901), ((512, 6144), 3.0, 902), ((96, 1024), 1.0, 903)]
    assert spg.lib.quantize_block16_path(6144, 8448) == 2
    assert spg.lib.quantize_block16_path(512, 6144) == 1 and spg.lib.quantize_block16_path(96, 1024) == 1
    ts = []
    for shape, std, seed in calls:
        x = dev(bf16_normal(shape, std, seed))
        ref = run(spg, x, noalloc=False, layout=layout)
        got = run(spg, x, noalloc=True, layout=layout)
        for a, b, what in zip(got, ref, ("codes", "block scales", "tensor scale")):
            assert np.array_equal(a, b), f"{shape} {layout}: {what} differ"
        ts.append(int(got[2][0]))
        del x
        torch.cuda.empty_cache()
    # every call's tensor scale is its own (a stale amax would repeat one)
    assert len(set(ts)) == 3
