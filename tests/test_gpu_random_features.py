"""Seeded random shapes with the optional features of gemm_scaled: bf16 and
E4M3 bias rows, outputs split into column segments (with a residual matrix
or a bias row), K-major operands, padded
leading dimensions, per-tensor batches (own or broadcast weights) and the
blocked NVFP4 scale planes.  Each case draws its shape and feature from a
fixed seed, runs quantize + GEMM on the device, and compares the whole output
with the oracle within the acceptance bound.
"""
import numpy as np
import pytest
import torch

import oracle
from synthetic import bf16_normal

pytestmark = pytest.mark.gpu

FEATURES = ["bias_bf16", "bias_e4m3", "split", "kmajor", "padded", "batch", "nvfp4_blocked", "split_bias"]


def _cases(per_feature=10, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for feat in FEATURES:
        for _ in range(per_feature):
            M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 200)), int(rng.integers(200, 600))]))
            if feat == "nvfp4_blocked":
                fmt, K = "nvfp4", int(rng.integers(1, 7)) * 256
            else:
                fmt = str(rng.choice(["e4m3_row", "e4m3_tensor"])) if feat != "batch" else "e4m3_tensor"
                K = int(rng.integers(1, 100)) * 16
            if feat in ("bias_bf16", "bias_e4m3", "split_bias"):
                epi = "add"
            else:
                epi = str(rng.choice(["store", "add", "swiglu"]))
            if feat in ("split", "split_bias"):
                n_out = int(rng.integers(2, 12)) * 64 + int(rng.integers(0, 64))
                N = 2 * n_out if epi == "swiglu" else n_out
            else:
                N = int(rng.integers(1, 450)) * 2
            out.append((feat, fmt, epi, M, N, K, int(rng.integers(0, 1 << 30))))
    return out


CASES = _cases()


def dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def kmajor_copy(codes, pad):
    """[.., R, K] codes stored K-major as [.., K, R] with a row stride of R
    rounded up to 16, plus pad."""
    t = codes.transpose(-1, -2)
    ld = (t.shape[-1] + 15) // 16 * 16 + pad
    buf = torch.zeros(t.shape[:-1] + (ld,), dtype=torch.uint8, device=codes.device)
    buf[..., : t.shape[-1]] = t
    return buf[..., : t.shape[-1]]


@pytest.fixture(scope="module")
def spg():
    import scaled_precision_gemm_amd as m
    return m


@pytest.mark.parametrize("feat,fmt,epi,M,N,K,seed", CASES, ids=lambda v: str(v))
def test_random_feature_matches_the_oracle(spg, feat, fmt, epi, M, N, K, seed):
    rng = np.random.default_rng(seed)
    B = 2 if feat == "batch" else 1
    own_w = feat == "batch" and bool(rng.integers(0, 2))
    n_out = N // 2 if epi == "swiglu" else N
    A16 = bf16_normal((B, M, K) if B > 1 else (M, K), 1.0, seed % 1000)
    W16 = bf16_normal((B, N, K) if own_w else (N, K), 0.02 if fmt == "e4m3_row" else 1.0, seed % 1000 + 1)
    R16 = bias16 = None
    bias_vals = None
    kw = {}
    if epi == "add" and feat not in ("bias_bf16", "bias_e4m3", "split_bias"):
        R16 = bf16_normal((M, n_out), 1.0, seed % 1000 + 2)
    if feat in ("bias_bf16", "split_bias"):
        bias16 = bf16_normal((n_out,), 1.0, seed % 1000 + 3)
        kw["residual"] = dev(bias16)
        bias_vals = oracle.bf16_to_f64(bias16)
    elif feat == "bias_e4m3":
        bias16 = bf16_normal((n_out,), 1.0, seed % 1000 + 3)
        padded = np.zeros((1, (n_out + 15) // 16 * 16), np.uint16)
        padded[0, :n_out] = bias16
        bq, bs = spg.quantize_rowwise(dev(padded))
        bq_o, bs_o = oracle.quantize_rowwise(bias16[None, :])
        kw["residual"], kw["bias_scale"] = bq[0, :n_out].contiguous(), bs
        bias_vals = oracle.bias_e4m3(bq_o[0], bs_o[0])
    elif R16 is not None:
        kw["residual"] = dev(R16)
    print(f"{feat} {fmt} {epi} B{B} {M}x{N}x{K} own_w={own_w}", flush=True)

    # device quantize (padded: codes written into rows of a wider buffer)
    A, W = dev(A16), dev(W16)
    if fmt == "e4m3_row":
        if feat == "padded":
            pad = 16 * int(rng.integers(1, 4))
            qa = torch.zeros((M, K + pad), dtype=torch.uint8, device="cuda")[:, :K]
            sa = torch.empty((M,), dtype=torch.float32, device="cuda")
            spg.quantize_rowwise(A, out=qa, scale=sa)
        else:
            qa, sa = spg.quantize_rowwise(A)
        qw, sw = spg.quantize_rowwise(W)
    elif fmt == "e4m3_tensor":
        qa, sa = spg.quantize_tensor(A)
        qw, sw = spg.quantize_tensor(W)
        if feat == "padded":
            pad = 16 * int(rng.integers(1, 4))
            buf = torch.zeros((M, K + pad), dtype=torch.uint8, device="cuda")
            buf[:, :K] = qa
            qa = buf[:, :K]
    else:
        qa, sa, ta = spg.quantize_block16(A, layout="blocked")
        qw, sw, tw = spg.quantize_block16(W, layout="blocked")
        kw.update(tscale_a=ta, tscale_w=tw, scale_layout="blocked")
    if feat == "kmajor":
        a_km, w_km = [(True, False), (False, True), (True, True)][int(rng.integers(0, 3))]
        if a_km:
            qa = kmajor_copy(qa, 16 * int(rng.integers(0, 3)))
        if w_km:
            qw = kmajor_copy(qw, 16 * int(rng.integers(0, 3)))
        kw.update(a_kmajor=a_km, w_kmajor=w_km)
    out = None
    if feat == "padded":
        ldo = (n_out + 7) // 8 * 8 + 8 * int(rng.integers(1, 4))
        out = torch.zeros((M, ldo), dtype=torch.bfloat16, device="cuda")[:, :n_out]
        kw["out"] = out
    if feat in ("split", "split_bias"):
        cuts = sorted(set(int(c) * 64 for c in rng.integers(1, n_out // 64 + 1, size=2) if int(c) * 64 < n_out))
        widths = [b - a for a, b in zip([0] + cuts, cuts + [n_out])]
        kw["out_split"] = widths
    res = spg.gemm_scaled(qa, sa, qw, sw, epi, fmt=fmt, **kw)
    if feat in ("split", "split_bias"):
        assert [t.shape[-1] for t in res] == widths
        got = np.concatenate([host(t) for t in res], axis=-1)
    else:
        got = host(out if out is not None else res)

    # oracle, per batch entry
    for b in range(B):
        Ab = A16[b] if B > 1 else A16
        Wb = W16[b] if own_w else W16
        if fmt == "e4m3_row":
            qa_o, sa_o = oracle.quantize_rowwise(Ab)
            qw_o, sw_o = oracle.quantize_rowwise(Wb)
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        elif fmt == "e4m3_tensor":
            qa_o, sa_o = oracle.quantize_tensor(Ab)
            qw_o, sw_o = oracle.quantize_tensor(Wb)
            sa_o, sw_o = sa_o[0], sw_o[0]
            D, Da = oracle.gemm_e4m3_sums(qa_o, qw_o)
        else:
            qa_o, ba_o, sa_o = oracle.quantize_block16(Ab)
            qw_o, bw_o, sw_o = oracle.quantize_block16(Wb)
            D, Da = oracle.gemm_nvfp4_sums(qa_o, ba_o, qw_o, bw_o)
        y, S, _ = oracle.epilogue(epi, D, Da, sa_o, sw_o, R16, bias_vals)
        g = got[b] if B > 1 else got
        assert g.shape == (M, n_out)
        ok, excess = oracle.within_tolerance(g, y, S)
        bad = np.argwhere(~ok)
        assert ok.all(), (f"batch {b}: {len(bad)} of {ok.size} outside the bound; worst excess "
                          f"{excess.max():.3g} at {bad[:5].tolist()}")
