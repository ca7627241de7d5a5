"""Quantize + GEMM captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library launches on the caller's stream, allocates nothing and
clears nothing with memset nodes, so a captured step replays like the eager
one.  Every route is covered (half-height tiles, the persistent kernel with
its ADD epilogue, split-K with its reduction through a workspace, the
decode-width kernel, per-tensor scales with their partial-maximum pass, and
NVFP4 with its two-pass quantizer).  Each replay runs on new input written
into the captured buffer, with eager work and synchronizations in between,
and must equal the eager result for that input bit for bit (the kernels are
deterministic).  Products launched on two streams at once must also equal the
same products run one after another.
"""
import numpy as np
import pytest
import torch

from synthetic import bf16_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spg():
    import scaled_precision_gemm_amd as m
    return m


def dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


CASES = [
    # (fmt, epilogue, M, N, K, batch, expected plan kernel)
    ("e4m3_row", "store", 300, 520, 1040, 1, 2),
    ("e4m3_row", "add", 2048, 8192, 512, 1, 0),
    ("e4m3_row", "add", 128, 5120, 4096, 1, 0),
    ("e4m3_row", "swiglu", 16, 4096, 1024, 1, 3),
    ("e4m3_tensor", "store", 512, 512, 512, 4, 2),
    ("nvfp4", "add", 256, 1024, 1024, 1, 1),
]


@pytest.mark.parametrize("fmt,epi,M,N,K,B,kernel", CASES,
                         ids=["half_tiles", "persistent_add", "split_k", "decode_width", "tensor_batch", "nvfp4"])
def test_captured_step_replays_like_eager(spg, fmt, epi, M, N, K, B, kernel):
    plan = spg.gemm_plan(M, N, K, fmt, epi, batch=B)
    assert plan["kernel"] == kernel
    if kernel == 0 and epi == "add" and M == 128:
        assert plan["split_k"] > 1
    n_out = N // 2 if epi == "swiglu" else N
    a_shape = (B, M, K) if B > 1 else (M, K)
    A = dev(bf16_normal(a_shape, 1.0, 500 + M))
    W = dev(bf16_normal((B, N, K) if B > 1 else (N, K), 0.02 if fmt != "e4m3_tensor" else 1.0, 501))
    R = dev(bf16_normal((M, n_out), 1.0, 502)) if epi == "add" else None
    if fmt == "e4m3_row":
        qw, sw = spg.quantize_rowwise(W)
    elif fmt == "e4m3_tensor":
        qw, sw = spg.quantize_tensor(W)
    else:
        qw, sw, tw = spg.quantize_block16(W)
    ws = None
    if plan["split_k"] > 1 or plan["tail_split"] > 1:
        a_codes = torch.empty(a_shape if fmt != "nvfp4" else (M, K // 2), dtype=torch.uint8, device="cuda")
        ws = spg.gemm_workspace(a_codes, qw, fmt, epi, residual=R)
        assert ws is not None and ws.numel() > 0

    def step():
        if fmt == "e4m3_row":
            qa, sa = spg.quantize_rowwise(A)
            return spg.gemm_scaled(qa, sa, qw, sw, epi, residual=R, workspace=ws)
        if fmt == "e4m3_tensor":
            qa, sa = spg.quantize_tensor(A)
            return spg.gemm_scaled(qa, sa, qw, sw, epi, fmt="e4m3_tensor", workspace=ws)
        qa, sa, ta = spg.quantize_block16(A)
        return spg.gemm_scaled(qa, sa, qw, sw, epi, residual=R, fmt="nvfp4", tscale_a=ta, tscale_w=tw,
                               workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_g = step()
    torch.cuda.synchronize()
    for r in range(3):
        A.copy_(dev(bf16_normal(a_shape, 1.0 + r, 600 + r)))
        want = host(step())                  # eager, on the same input
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(out_g)
        assert np.array_equal(got, want), f"replay {r}: {np.count_nonzero(got != want)} elements differ"
        torch.cuda.synchronize()


def test_two_streams_at_once_match_one_stream(spg):
    # the library keeps no state between calls (each call's workspace is its
    # own): products launched on two streams at once give the results they
    # give one after another on one stream, bit for bit
    shapes = [("e4m3_row", "add", 128, 5120, 4096), ("e4m3_row", "swiglu", 300, 2048, 1536),
              ("nvfp4", "store", 256, 1024, 1024), ("e4m3_row", "store", 16, 4096, 2048)]
    inputs = []
    for i, (fmt, epi, M, N, K) in enumerate(shapes):
        A = dev(bf16_normal((M, K), 1.0, 900 + i))
        W = dev(bf16_normal((N, K), 0.02, 910 + i))
        n_out = N // 2 if epi == "swiglu" else N
        R = dev(bf16_normal((M, n_out), 1.0, 920 + i)) if epi == "add" else None
        inputs.append((fmt, epi, A, W, R))

    def run(fmt, epi, A, W, R):
        if fmt == "nvfp4":
            qa, sa, ta = spg.quantize_block16(A)
            qw, sw, tw = spg.quantize_block16(W)
            return spg.gemm_scaled(qa, sa, qw, sw, epi, residual=R, fmt="nvfp4", tscale_a=ta, tscale_w=tw)
        qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
        return spg.gemm_scaled(qa, sa, qw, sw, epi, residual=R)

    want = [host(run(*x)) for x in inputs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [None] * len(inputs)
    for rep in range(3):
        for i, x in enumerate(inputs):
            with torch.cuda.stream(streams[i % 2]):
                got[i] = run(*x)
        torch.cuda.synchronize()
        for i in range(len(inputs)):
            assert np.array_equal(host(got[i]), want[i]), f"round {rep}, product {i}"
