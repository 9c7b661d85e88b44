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

Each op calls the binding (one kernel on the current stream) and has a fake
implementation giving output shapes and dtypes, so the ops stay opaque to
the compiler, as the vLLM API page "vllm.kernels.aiter_ops" describes for
its aiter_lib fragment of wrapped AITER ops.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (FP8_DTYPE, fused_add_rmsnorm, fused_add_rmsnorm_fp8, rmsnorm, rmsnorm_fp8,
               silu_and_mul, silu_and_mul_fp8)

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
