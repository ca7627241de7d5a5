"""quantize_block16_noalloc through the C ABI against quantize_block16.

The allocation-free variant keeps its scratch (partial maxima of the tensor
amax) in a static device array shared by every call on the GPU.  Two calls
in a row: the second has fewer partial maxima than the first and a smaller
amax, so a stale partial left in the array by the first call would change
the second call's tensor scale.  Codes, block scales and the tensor scale
must equal the workspace entry point's bit for bit.
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


def run(spg, x, noalloc):
    R, K = x.shape
    q = torch.full((R, K // 2), 0xA5, dtype=torch.uint8, device="cuda")
    bs = torch.full((R, K // 16), 0x5A, dtype=torch.uint8, device="cuda")
    t = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda a: ctypes.c_void_p(a.data_ptr())
    if noalloc:
        st = spg.lib.quantize_block16_noalloc(P(x), R, K, P(q), P(bs), P(t), stream)
    else:
        nws = spg.lib.quantize_block16_workspace_bytes(R, K)
        ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device="cuda")
        st = spg.lib.quantize_block16(P(x), R, K, P(q), P(bs), P(t), P(ws), ws.numel(), stream)
    assert st == 0, spg.lib.spg_status_string(st)
    torch.cuda.synchronize()
    return q.cpu().numpy(), bs.cpu().numpy(), t.cpu().numpy().view(np.uint32)


def test_noalloc_matches_workspace_entry_point_on_two_calls(spg):
    big = bf16_normal((512, 6144), 10.0, 901)      # 192 partial maxima, amax ~ 50
    small = bf16_normal((96, 1024), 1.0, 902)      # 6 partial maxima, amax ~ 4.5
    for x16 in (big, small):
        x = dev(x16)
        ref = run(spg, x, noalloc=False)
        got = run(spg, x, noalloc=True)
        for a, b, what in zip(got, ref, ("codes", "block scales", "tensor scale")):
            assert np.array_equal(a, b), f"{x16.shape}: {what} differ"
    # and the small call's tensor scale is its own, not the big call's
    assert ref[2][0] != run(spg, dev(big), noalloc=False)[2][0]
