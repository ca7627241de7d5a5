"""The Python binding's argument checks (CPU only, nothing is launched).

Tensors live on torch's "meta" device: they carry shapes, strides and dtypes
but no memory, so each call below stops at the check it is meant to trip, a
ValueError raised before the library is called.  A call that passes every
check ends at the request for CUDA tensors.
"""
import pytest
import torch

import scaled_precision_gemm_amd as spg

M, N, K = 64, 96, 128


def t(shape, dtype, device="meta"):
    return torch.empty(shape, dtype=dtype, device=device)


def row_args(**over):
    a = dict(A=t((M, K), torch.uint8), sa=t((M,), torch.float32), W=t((N, K), torch.uint8),
             sw=t((N,), torch.float32), epilogue="store", residual=None, fmt="e4m3_row", out=None)
    a.update(over)
    return a


def call(a):
    return spg.gemm_scaled(a.pop("A"), a.pop("sa"), a.pop("W"), a.pop("sw"), **a)


def test_valid_call_reaches_the_device_check():
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args())
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(epilogue="add", residual=t((M, N), torch.bfloat16), out=t((M, N), torch.bfloat16)))
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(epilogue="add", residual=t((N,), torch.bfloat16)))
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(epilogue="swiglu", out=t((M, N // 2), torch.bfloat16)))
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(epilogue="add", residual=t((N,), torch.uint8), bias_scale=t((1,), torch.float32)))
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(out_split=[64, N - 64]))
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(A=t((K, M), torch.uint8), W=t((K, N), torch.uint8), a_kmajor=True, w_kmajor=True))
    with pytest.raises(ValueError, match="CUDA"):
        call(row_args(out_split=[t((M, 64), torch.bfloat16), t((M, N - 64), torch.bfloat16)]))


@pytest.mark.parametrize("case,match", [
    ("out_2d_for_batched", "out must have shape"),
    ("out_wrong_shape", "out must have shape"),
    ("out_strided_rows", "rows of out"),
    ("out_fp32", "out must be bf16"),
    ("residual_small", "residual must have one of the shapes"),
    ("residual_strided", "rows of the residual"),
    ("residual_for_store", "only by the add epilogue"),
    ("add_without_residual", "needs a residual"),
    ("sa_short", "sa must hold"),
    ("sw_fp16", "row scales must be fp32"),
    ("tensor_scale_count", "sa must hold"),
    ("nvfp4_plane_shape", "sa must be a contiguous"),
    ("nvfp4_no_tscale", "tscale_a must be one fp32 value"),
    ("other_device", "must be on meta"),
    ("a_strided", "rows of A and W"),
    ("k_mismatch", "disagree on K"),
    ("bias_scale_for_store", "bias scale is taken only by the add"),
    ("bias_scale_with_bf16_row", "E4M3 codes"),
    ("bias_scale_with_matrix", "E4M3 codes"),
    ("bias_scale_two_values", "bias_scale must be one fp32 value"),
    ("codes_without_bias_scale", "residual must be bf16"),
    ("split_and_out", "exclusive"),
    ("split_widths_sum", "adding up to"),
    ("split_boundary", "multiple of 64"),
    ("split_tensor_dtype", "must be a bf16 tensor"),
    ("split_tensor_rows", "wrong rows"),
    ("split_tensor_stride", "row stride a multiple of 8"),
    ("kmajor_nvfp4", "only by the FP8 formats"),
    ("kmajor_k_mismatch", "disagree on K"),
])
def test_bad_calls_raise_before_the_library(case, match):
    a = row_args()
    if case == "out_2d_for_batched":
        a.update(fmt="e4m3_tensor", A=t((2, M, K), torch.uint8), sa=t((2,), torch.float32),
                 sw=t((1,), torch.float32), out=t((M, N), torch.bfloat16))
    elif case == "out_wrong_shape":
        a["out"] = t((M, N - 1), torch.bfloat16)
    elif case == "out_strided_rows":
        a["out"] = t((N, M), torch.bfloat16).t()
    elif case == "out_fp32":
        a["out"] = t((M, N), torch.float32)
    elif case == "residual_small":
        a.update(epilogue="add", residual=t((M - 1, N), torch.bfloat16))
    elif case == "residual_strided":
        a.update(epilogue="add", residual=t((N, M), torch.bfloat16).t())
    elif case == "residual_for_store":
        a["residual"] = t((M, N), torch.bfloat16)
    elif case == "add_without_residual":
        a["epilogue"] = "add"
    elif case == "sa_short":
        a["sa"] = t((M - 1,), torch.float32)
    elif case == "sw_fp16":
        a["sw"] = t((N,), torch.float16)
    elif case == "tensor_scale_count":
        a.update(fmt="e4m3_tensor", sa=t((M,), torch.float32), sw=t((1,), torch.float32))
    elif case == "nvfp4_plane_shape":
        a.update(fmt="nvfp4", A=t((M, K // 2), torch.uint8), W=t((N, K // 2), torch.uint8),
                 sa=t((M, K // 32), torch.uint8), sw=t((N, K // 16), torch.uint8),
                 tscale_a=t((1,), torch.float32), tscale_w=t((1,), torch.float32))
    elif case == "nvfp4_no_tscale":
        a.update(fmt="nvfp4", A=t((M, K // 2), torch.uint8), W=t((N, K // 2), torch.uint8),
                 sa=t((M, K // 16), torch.uint8), sw=t((N, K // 16), torch.uint8))
    elif case == "other_device":
        a["sw"] = t((N,), torch.float32, device="cpu")
    elif case == "a_strided":
        a["A"] = t((K, M), torch.uint8).t()
    elif case == "k_mismatch":
        a["W"] = t((N, K + 16), torch.uint8)
    elif case == "bias_scale_for_store":
        a.update(bias_scale=t((1,), torch.float32))
    elif case == "bias_scale_with_bf16_row":
        a.update(epilogue="add", residual=t((N,), torch.bfloat16), bias_scale=t((1,), torch.float32))
    elif case == "bias_scale_with_matrix":
        a.update(epilogue="add", residual=t((M, N), torch.uint8), bias_scale=t((1,), torch.float32))
    elif case == "bias_scale_two_values":
        a.update(epilogue="add", residual=t((N,), torch.uint8), bias_scale=t((2,), torch.float32))
    elif case == "codes_without_bias_scale":
        a.update(epilogue="add", residual=t((N,), torch.uint8))
    elif case == "split_and_out":
        a.update(out=t((M, N), torch.bfloat16), out_split=[64, N - 64])
    elif case == "split_widths_sum":
        a.update(out_split=[64, N - 63])
    elif case == "split_boundary":
        a.update(out_split=[32, N - 32])
    elif case == "split_tensor_dtype":
        a.update(out_split=[t((M, 64), torch.bfloat16), t((M, N - 64), torch.float16)])
    elif case == "split_tensor_rows":
        a.update(out_split=[t((M, 64), torch.bfloat16), t((M + 1, N - 64), torch.bfloat16)])
    elif case == "kmajor_nvfp4":
        a.update(fmt="nvfp4", A=t((M, K // 2), torch.uint8), W=t((N, K // 2), torch.uint8),
                 sa=t((M, K // 16), torch.uint8), sw=t((N, K // 16), torch.uint8),
                 tscale_a=t((1,), torch.float32), tscale_w=t((1,), torch.float32), w_kmajor=True)
    elif case == "kmajor_k_mismatch":
        a.update(W=t((K + 16, N), torch.uint8), w_kmajor=True)
    elif case == "split_tensor_stride":
        a.update(out_split=[t((M, 68), torch.bfloat16)[:, :64], t((M, N - 64), torch.bfloat16)])
    with pytest.raises(ValueError, match=match):
        call(a)
