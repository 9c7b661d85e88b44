"""torch custom ops over the library, for callers behind torch.compile.

Importing this module registers, in the ``arn`` namespace:

    arn::rmsnorm(x, weight, eps) -> y
    arn::fused_add_rmsnorm(x, residual!, weight, eps) -> y          (residual updated)
    arn::rmsnorm_fp8_static(x, weight, eps, scale) -> codes
    arn::rmsnorm_fp8_dynamic(x, weight, eps) -> (codes, scales)
    arn::fused_add_rmsnorm_fp8_static(x, residual!, weight, eps, scale) -> codes
    arn::fused_add_rmsnorm_fp8_dynamic(x, residual!, weight, eps) -> (codes, scales)
    arn::silu_and_mul(x) -> y
    arn::silu_and_mul_fp8_static(x, scale) -> codes
    arn::silu_and_mul_fp8_dynamic(x) -> (codes, scales)
    arn::sum_add_rmsnorm(parts[], residual!, weight, eps) -> y           (residual updated)
    arn::sum_add_rmsnorm_fp8_dynamic(parts[], residual!, weight, eps) -> (codes, scales)
    arn::fp8_weight_preshuffle(b) -> shuffled weight bytes
    arn::fp8_gemm(a, scale_a, b, scale_b, out_dtype) -> c
    arn::fp8_gemm_preshuffled(a, scale_a, b_shuffled, n, k, scale_b, out_dtype) -> c

Each op calls the binding (one kernel on the current stream) and has a fake
implementation giving output shapes and dtypes, so the ops stay opaque to
the compiler, as the vLLM API page "vllm.kernels.aiter_ops" describes for
its aiter_lib fragment of wrapped AITER ops.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (FP8_DTYPE, PreshuffledWeight, fp8_gemm, fp8_weight_preshuffle, fused_add_rmsnorm,
               fused_add_rmsnorm_fp8, rmsnorm, rmsnorm_fp8, silu_and_mul, silu_and_mul_fp8,
               sum_add_rmsnorm)

Tensor = torch.Tensor


def _scales_like(x: Tensor) -> Tensor:
    return torch.empty(x.shape[:-1] if x.dim() > 1 else (1,), dtype=torch.float32,
                       device=x.device)


def _glu_shape(x: Tensor):
    return (*x.shape[:-1], x.shape[-1] // 2)


@torch.library.custom_op("arn::rmsnorm", mutates_args=())
def rmsnorm_op(x: Tensor, weight: Optional[Tensor], eps: float) -> Tensor:
    return rmsnorm(x, weight, eps)


@rmsnorm_op.register_fake
def _(x, weight, eps):
    return torch.empty_like(x)


@torch.library.custom_op("arn::fused_add_rmsnorm", mutates_args=("residual",))
def fused_add_rmsnorm_op(x: Tensor, residual: Tensor, weight: Optional[Tensor],
                         eps: float) -> Tensor:
    return fused_add_rmsnorm(x, residual, weight, eps)


@fused_add_rmsnorm_op.register_fake
def _(x, residual, weight, eps):
    return torch.empty_like(x)


@torch.library.custom_op("arn::rmsnorm_fp8_static", mutates_args=())
def rmsnorm_fp8_static_op(x: Tensor, weight: Optional[Tensor], eps: float,
                          scale: Tensor) -> Tensor:
    return rmsnorm_fp8(x, weight, eps, scale=scale)[0]


@rmsnorm_fp8_static_op.register_fake
def _(x, weight, eps, scale):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device)


@torch.library.custom_op("arn::rmsnorm_fp8_dynamic", mutates_args=())
def rmsnorm_fp8_dynamic_op(x: Tensor, weight: Optional[Tensor],
                           eps: float) -> tuple[Tensor, Tensor]:
    q, s = rmsnorm_fp8(x, weight, eps, dynamic=True)
    return q, s


@rmsnorm_fp8_dynamic_op.register_fake
def _(x, weight, eps):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device), _scales_like(x)


@torch.library.custom_op("arn::fused_add_rmsnorm_fp8_static", mutates_args=("residual",))
def fused_add_rmsnorm_fp8_static_op(x: Tensor, residual: Tensor, weight: Optional[Tensor],
                                    eps: float, scale: Tensor) -> Tensor:
    return fused_add_rmsnorm_fp8(x, residual, weight, eps, scale=scale)[0]


@fused_add_rmsnorm_fp8_static_op.register_fake
def _(x, residual, weight, eps, scale):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device)


@torch.library.custom_op("arn::fused_add_rmsnorm_fp8_dynamic", mutates_args=("residual",))
def fused_add_rmsnorm_fp8_dynamic_op(x: Tensor, residual: Tensor, weight: Optional[Tensor],
                                     eps: float) -> tuple[Tensor, Tensor]:
    q, s = fused_add_rmsnorm_fp8(x, residual, weight, eps, dynamic=True)
    return q, s


@fused_add_rmsnorm_fp8_dynamic_op.register_fake
def _(x, residual, weight, eps):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device), _scales_like(x)


@torch.library.custom_op("arn::silu_and_mul", mutates_args=())
def silu_and_mul_op(x: Tensor) -> Tensor:
    return silu_and_mul(x)


@silu_and_mul_op.register_fake
def _(x):
    return torch.empty(_glu_shape(x), dtype=x.dtype, device=x.device)


@torch.library.custom_op("arn::silu_and_mul_fp8_static", mutates_args=())
def silu_and_mul_fp8_static_op(x: Tensor, scale: Tensor) -> Tensor:
    return silu_and_mul_fp8(x, scale=scale)[0]


@silu_and_mul_fp8_static_op.register_fake
def _(x, scale):
    return torch.empty(_glu_shape(x), dtype=FP8_DTYPE, device=x.device)


@torch.library.custom_op("arn::silu_and_mul_fp8_dynamic", mutates_args=())
def silu_and_mul_fp8_dynamic_op(x: Tensor) -> tuple[Tensor, Tensor]:
    q, s = silu_and_mul_fp8(x, dynamic=True)
    return q, s


@silu_and_mul_fp8_dynamic_op.register_fake
def _(x):
    return torch.empty(_glu_shape(x), dtype=FP8_DTYPE, device=x.device), _scales_like(x)


def _preshuffled_bytes(n: int, k: int) -> int:
    # ceil(n / 16) column tiles x ceil(k / 128) k steps of 2 KiB (arn.h)
    return max(((n + 15) // 16) * ((k + 127) // 128) * 2048, 16)


@torch.library.custom_op("arn::fp8_weight_preshuffle", mutates_args=())
def fp8_weight_preshuffle_op(b: Tensor) -> Tensor:
    return fp8_weight_preshuffle(b).data


@fp8_weight_preshuffle_op.register_fake
def _(b):
    return torch.empty(_preshuffled_bytes(b.shape[0], b.shape[1]), dtype=torch.uint8,
                       device=b.device)


@torch.library.custom_op("arn::fp8_gemm", mutates_args=())
def fp8_gemm_op(a: Tensor, scale_a: Tensor, b: Tensor, scale_b: Tensor,
                out_dtype: torch.dtype = torch.bfloat16) -> Tensor:
    return fp8_gemm(a, scale_a, b, scale_b, out_dtype=out_dtype)


@fp8_gemm_op.register_fake
def _(a, scale_a, b, scale_b, out_dtype=torch.bfloat16):
    return torch.empty((a.shape[0], b.shape[0]), dtype=out_dtype, device=a.device)


@torch.library.custom_op("arn::fp8_gemm_preshuffled", mutates_args=())
def fp8_gemm_preshuffled_op(a: Tensor, scale_a: Tensor, b_shuffled: Tensor, n: int, k: int,
                            scale_b: Tensor, out_dtype: torch.dtype = torch.bfloat16) -> Tensor:
    if b_shuffled.numel() < _preshuffled_bytes(n, k):
        raise ValueError("b_shuffled is smaller than a pre-shuffled n x k weight")
    return fp8_gemm(a, scale_a, PreshuffledWeight(b_shuffled, n, k), scale_b,
                    out_dtype=out_dtype)


@fp8_gemm_preshuffled_op.register_fake
def _(a, scale_a, b_shuffled, n, k, scale_b, out_dtype=torch.bfloat16):
    return torch.empty((a.shape[0], n), dtype=out_dtype, device=a.device)


@torch.library.custom_op("arn::sum_add_rmsnorm", mutates_args=("residual",))
def sum_add_rmsnorm_op(parts: list[Tensor], residual: Tensor, weight: Optional[Tensor],
                       eps: float) -> Tensor:
    return sum_add_rmsnorm(parts, weight, eps, residual=residual)


@sum_add_rmsnorm_op.register_fake
def _(parts, residual, weight, eps):
    return torch.empty_like(parts[0])


@torch.library.custom_op("arn::sum_add_rmsnorm_fp8_dynamic", mutates_args=("residual",))
def sum_add_rmsnorm_fp8_dynamic_op(parts: list[Tensor], residual: Tensor,
                                   weight: Optional[Tensor], eps: float) -> tuple[Tensor, Tensor]:
    q, s = sum_add_rmsnorm(parts, weight, eps, residual=residual, fp8="dynamic")
    return q, s


@sum_add_rmsnorm_fp8_dynamic_op.register_fake
def _(parts, residual, weight, eps):
    x = parts[0]
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device), _scales_like(x)
