"""The torch custom ops register and give the right shapes and dtypes
through their fake implementations (no GPU needed)."""
import torch
from torch._subclasses.fake_tensor import FakeTensorMode

import residual_add_rmsnorm_amd.torch_ops  # noqa: F401  (registers arn::*)

OPS = ["rmsnorm", "fused_add_rmsnorm", "rmsnorm_fp8_static", "rmsnorm_fp8_dynamic",
       "fused_add_rmsnorm_fp8_static", "fused_add_rmsnorm_fp8_dynamic", "silu_and_mul",
       "silu_and_mul_fp8_static", "silu_and_mul_fp8_dynamic", "fp8_weight_preshuffle",
       "fp8_gemm", "fp8_gemm_preshuffled", "sum_add_rmsnorm", "sum_add_rmsnorm_fp8_dynamic"]


def test_ops_registered():
    for name in OPS:
        assert hasattr(torch.ops.arn, name), name


def test_fake_shapes():
    with FakeTensorMode():
        x = torch.empty(4, 7, 96, dtype=torch.bfloat16)
        r = torch.empty_like(x)
        w = torch.empty(96, dtype=torch.bfloat16)
        s = torch.empty(1, dtype=torch.float32)
        assert torch.ops.arn.rmsnorm(x, w, 1e-6).shape == x.shape
        assert torch.ops.arn.fused_add_rmsnorm(x, r, w, 1e-6).dtype == torch.bfloat16
        q = torch.ops.arn.rmsnorm_fp8_static(x, w, 1e-6, s)
        assert q.shape == x.shape and q.dtype == torch.float8_e4m3fn
        q, sc = torch.ops.arn.fused_add_rmsnorm_fp8_dynamic(x, r, None, 1e-6)
        assert q.shape == x.shape and sc.shape == (4, 7) and sc.dtype == torch.float32
        g = torch.empty(5, 2 * 48, dtype=torch.float16)
        assert torch.ops.arn.silu_and_mul(g).shape == (5, 48)
        q, sc = torch.ops.arn.silu_and_mul_fp8_dynamic(g)
        assert q.shape == (5, 48) and sc.shape == (5,)
        b = torch.empty(40, 48, dtype=torch.float8_e4m3fn)
        sb = torch.empty(40, dtype=torch.float32)
        c = torch.ops.arn.fp8_gemm(q, sc, b, sb)
        assert c.shape == (5, 40) and c.dtype == torch.bfloat16
        bs = torch.ops.arn.fp8_weight_preshuffle(b)
        assert bs.shape == (3 * 1 * 2048,) and bs.dtype == torch.uint8
        c = torch.ops.arn.fp8_gemm_preshuffled(q, sc, bs, 40, 48, sb, torch.float16)
        assert c.shape == (5, 40) and c.dtype == torch.float16
        y = torch.ops.arn.sum_add_rmsnorm([x, x, x], r, w, 1e-6)
        assert y.shape == x.shape and y.dtype == x.dtype
        q, sc = torch.ops.arn.sum_add_rmsnorm_fp8_dynamic([x, x], r, w, 1e-6)
        assert q.dtype == torch.float8_e4m3fn and sc.shape == (4, 7)
