"""The measurement probes bench.py quotes (MFMA-only rate with its shader
clock, HBM read stream): their outputs are well formed and the read probe
really reads every byte of its buffer (its XOR fold matches the host's)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def spg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import scaled_precision_gemm_amd as m
    return m


@pytest.mark.parametrize("kind", [0, 1], ids=["fp8", "f16"])
def test_probe_mfma(spg, kind):
    sink, clocks, flops = spg.probe_mfma(kind, 200, 8)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    c = clocks.cpu().tolist()
    assert s.shape == (8 * 256,) and np.all(np.isfinite(s))
    assert c[1] > c[0] and c[3] > c[2]
    sclk_ghz = (c[1] - c[0]) / (c[3] - c[2]) * 0.1
    assert 0.3 < sclk_ghz < 3.5
    assert flops == 8 * 4 * 200 * 4 * (131072 if kind == 0 else 32768)
    sink2, _, _ = spg.probe_mfma(kind, 200, 8)        # same operands, same sums
    torch.cuda.synchronize()
    assert np.array_equal(sink2.cpu().numpy(), s)


@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096 + 48, 3), (1 << 24, 64)])
def test_probe_read_covers_the_buffer(spg, nbytes, wgs):
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    sink = spg.probe_read(host.cuda(), wgs)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want



def test_gemm_clock_probe_records_the_kernel_clock(spg):
    # the optional clock record of gemm_scaled's main launch: counters move
    # forward, the implied shader clock is plausible, and the output does not
    # depend on it
    from synthetic import bf16_normal
    A = torch.from_numpy(bf16_normal((1024, 1024), 1.0, 5).view(np.int16)).view(torch.bfloat16).cuda()
    W = torch.from_numpy(bf16_normal((2048, 1024), 0.02, 6).view(np.int16)).view(torch.bfloat16).cuda()
    qa, sa = spg.quantize_rowwise(A)
    qw, sw = spg.quantize_rowwise(W)
    clk = torch.zeros(4, dtype=torch.int64, device="cuda")
    out1 = spg.gemm_scaled(qa, sa, qw, sw, "swiglu", clock_probe=clk)
    out2 = spg.gemm_scaled(qa, sa, qw, sw, "swiglu")
    torch.cuda.synchronize()
    c = clk.cpu().numpy().astype(np.float64)
    assert c[1] > c[0] and c[3] > c[2]
    assert 0.3 < (c[1] - c[0]) / (c[3] - c[2]) / 10.0 < 3.5
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
