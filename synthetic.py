"""Seeded synthetic inputs, shared by the tests, smoke() and bench.py.

This module holds data generation only: no quantization, GEMM or epilogue
arithmetic.  Values are drawn from numpy's PCG64 generator (standard normal,
float32), scaled by the stated standard deviation, and rounded to bf16 with
round-to-nearest-even.  bf16 arrays are returned as ``np.uint16`` bit
patterns.

The workloads mirror the shapes the source pages measure (ninfer PR #167's
operator table, ninfer PR #160's T=4096 NVFP4 table, the AstrAI commit log's
L20 benchmark list): activations ~ N(0, 1), weights ~ N(0, 0.02), residuals
~ N(0, 1).  The pages measured real model activations and trained weights;
these seeded normals stand in for them.
"""
from __future__ import annotations

import dataclasses

import numpy as np


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_normal(shape, std: float, seed: int) -> np.ndarray:
    """bf16 bits of shape ``shape`` drawn from N(0, std^2) with a fixed seed."""
    n = int(np.prod(shape))
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=n, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x).reshape(shape)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One GEMM workload: out = epilogue(scale * A @ W^T)."""
    name: str
    fmt: str            # "e4m3_row", "e4m3_tensor" or "nvfp4"
    epilogue: str       # "store", "add" or "swiglu"
    M: int              # tokens (rows of A)
    N: int              # weight rows (for swiglu: gate rows then up rows)
    K: int
    batch: int = 1
    a_std: float = 1.0
    w_std: float = 0.02
    seed: int = 0
    bias: bool = False  # "add" with one bf16 row [n_out] (a bias) instead of an [M, n_out] residual
    split: tuple = ()   # output column widths of a split-N output (one tensor per segment), else one output

    @property
    def n_out(self) -> int:
        return self.N // 2 if self.epilogue == "swiglu" else self.N

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    def a_shape(self):
        return (self.batch, self.M, self.K) if self.batch > 1 else (self.M, self.K)

    def w_shape(self):
        return (self.batch, self.N, self.K) if self.batch > 1 else (self.N, self.K)

    def inputs(self, rows_a=None):
        """(A, W, residual-or-None) as bf16 bits, seeds 100c+1/2/3."""
        A = bf16_normal(self.a_shape(), self.a_std, self.seed + 1)
        W = bf16_normal(self.w_shape(), self.w_std, self.seed + 2)
        R = None
        if self.epilogue == "add":
            R = bf16_normal((self.n_out,) if self.bias else (self.M, self.n_out), 1.0, self.seed + 3)
        return A, W, R


WORKLOADS = {
    # tiny row-scaled FP8 GEMM, plain store
    "fp8_row_tiny": Workload("fp8_row_tiny", "e4m3_row", "store", 128, 256, 512, seed=100),
    # down-projection linear_add at T=1024: [N=5120, K=17408]
    "fp8_row_add_t1024": Workload("fp8_row_add_t1024", "e4m3_row", "add", 1024, 5120, 17408, seed=200),
    # fused gate/up SwiGLU at T=4096: W [34816, 5120] = gate rows then up rows
    "fp8_row_swiglu_t4096": Workload("fp8_row_swiglu_t4096", "e4m3_row", "swiglu", 4096, 34816, 5120, seed=300),
    # NVFP4 linear_add at T=4096: [N=5120, K=6144]
    "nvfp4_add_t4096": Workload("nvfp4_add_t4096", "nvfp4", "add", 4096, 5120, 6144, seed=400),
    # per-tensor FP8 batch of 64 512^3 products, and one 8192^3 product
    "fp8_tensor_bmm64_512": Workload("fp8_tensor_bmm64_512", "e4m3_tensor", "store", 512, 512, 512,
                                     batch=64, w_std=1.0, seed=500),
    "fp8_tensor_square_8192": Workload("fp8_tensor_square_8192", "e4m3_tensor", "store", 8192, 8192, 8192,
                                       w_std=1.0, seed=510),
    # the same two FP8 linears at 16 tokens (the narrow, weight-streaming route)
    "fp8_row_add_t16": Workload("fp8_row_add_t16", "e4m3_row", "add", 16, 5120, 17408, seed=600),
    "fp8_row_swiglu_t16": Workload("fp8_row_swiglu_t16", "e4m3_row", "swiglu", 16, 34816, 5120, seed=610),
    # the NVFP4 [N=5120, K=6144] linear and the [34816, 5120] gate/up at 16 tokens
    "nvfp4_add_t16": Workload("nvfp4_add_t16", "nvfp4", "add", 16, 5120, 6144, seed=620),
    "nvfp4_swiglu_t16": Workload("nvfp4_swiglu_t16", "nvfp4", "swiglu", 16, 34816, 5120, seed=630),
    # the T=4096 [N=5120, K=6144] linear in row-scaled FP8 with a fused bf16 bias row
    "fp8_row_bias_t4096": Workload("fp8_row_bias_t4096", "e4m3_row", "add", 4096, 5120, 6144, seed=700, bias=True),
    # fused input projections with split outputs (the pages name the call
    # sites, attn_input_proj and gdn_input_proj, but give no shapes): an
    # attention q | k | v projection with 40 query and 8 key/value heads of
    # 128 from a 5120-wide hidden state, and a gated-delta-net q | k | v | z
    # projection (16 + 16 key heads and 32 + 32 value heads of 128) from 2048
    "fp8_row_attn_in_t4096": Workload("fp8_row_attn_in_t4096", "e4m3_row", "store", 4096, 7168, 5120, seed=800,
                                      split=(5120, 1024, 1024)),
    "fp8_row_gdn_in_t4096": Workload("fp8_row_gdn_in_t4096", "e4m3_row", "store", 4096, 12288, 2048, seed=810,
                                     split=(2048, 2048, 4096, 4096)),
}
