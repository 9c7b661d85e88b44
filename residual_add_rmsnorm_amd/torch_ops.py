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
    arn::fp8_gemm(a, scale_a, b, scale_b, out_dtype=None) -> c        (None: bfloat16)
    arn::fp8_gemm_preshuffled(a, scale_a, b_shuffled, n, k, scale_b, out_dtype=None) -> c

Each op launches one kernel of the library on the current stream and has a
fake implementation giving output shapes and dtypes, so the ops stay opaque
to the compiler, as the vLLM API page "vllm.kernels.aiter_ops" describes for
its aiter_lib fragment of wrapped AITER ops.  The norm, SwiGLU and GEMM ops
are defined in C++ (csrc/arn_pyext.cpp, CUDA dispatch key) with the
binding's checks; the weight shuffle and the all-reduce form are Python
custom ops over the binding.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import FP8_DTYPE, _lib, fp8_weight_preshuffle, sum_add_rmsnorm

Tensor = torch.Tensor


def _scales_like(x: Tensor) -> Tensor:
    return torch.empty(x.shape[:-1] if x.dim() > 1 else (1,), dtype=torch.float32,
                       device=x.device)


def _glu_shape(x: Tensor):
    return (*x.shape[:-1], x.shape[-1] // 2)


# The ops of a decode step are defined and implemented in C++ (the binding's
# extension module, for the CUDA dispatch key), so an eager call through
# torch.ops reaches the library without running Python; loading the module
# registers them.  Their fakes follow.
_lib.native()


@torch.library.register_fake("arn::rmsnorm")
def _(x, weight, eps):
    return torch.empty_like(x)


@torch.library.register_fake("arn::fused_add_rmsnorm")
def _(x, residual, weight, eps):
    return torch.empty_like(x)


@torch.library.register_fake("arn::rmsnorm_fp8_static")
def _(x, weight, eps, scale):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device)


@torch.library.register_fake("arn::rmsnorm_fp8_dynamic")
def _(x, weight, eps):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device), _scales_like(x)


@torch.library.register_fake("arn::fused_add_rmsnorm_fp8_static")
def _(x, residual, weight, eps, scale):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device)


@torch.library.register_fake("arn::fused_add_rmsnorm_fp8_dynamic")
def _(x, residual, weight, eps):
    return torch.empty(x.shape, dtype=FP8_DTYPE, device=x.device), _scales_like(x)


@torch.library.register_fake("arn::silu_and_mul")
def _(x):
    return torch.empty(_glu_shape(x), dtype=x.dtype, device=x.device)


@torch.library.register_fake("arn::silu_and_mul_fp8_static")
def _(x, scale):
    return torch.empty(_glu_shape(x), dtype=FP8_DTYPE, device=x.device)


@torch.library.register_fake("arn::silu_and_mul_fp8_dynamic")
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


@torch.library.register_fake("arn::fp8_gemm")
def _(a, scale_a, b, scale_b, out_dtype=None):
    return torch.empty((a.shape[0], b.shape[0]), dtype=out_dtype or torch.bfloat16,
                       device=a.device)


@torch.library.register_fake("arn::fp8_gemm_preshuffled")
def _(a, scale_a, b_shuffled, n, k, scale_b, out_dtype=None):
    return torch.empty((a.shape[0], n), dtype=out_dtype or torch.bfloat16, device=a.device)


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
