"""Fused residual-add + RMSNorm (+ OCP e4m3) for AMD Instinct MI355X (gfx950),
with the SwiGLU + e4m3 activation and the e4m3 GEMM that consume its codes.

A thin binding over the C ABI of libarn.so (include/arn.h): each function
checks and marshals torch tensors into (device pointer, row stride) pairs and
calls the C entry point of the same name on torch's current stream.  For the
per-step calls (the norm forms, SwiGLU, the GEMM) that marshalling runs in
the extension module lib/_native (csrc/arn_pyext.cpp), since in Python it
would cost more host time than a decode-sized kernel takes.  Every step of
the operator runs in the library's HIP kernels; there is no fallback.  torch
provides device memory and streams only.

Layouts follow the vLLM API page "vllm.kernels.aiter_ops"
(flatten_to_2d_is_free): the last dimension must have unit stride and the
leading dimensions must flatten to rows with one uniform pitch without a
copy.  A padded pitch (row stride > hidden) is accepted; anything that
would need a copy raises ValueError instead of copying.
"""
from __future__ import annotations

import contextlib

import torch

from . import _lib
from ._lib import ArnError  # noqa: F401

__all__ = [
    "rmsnorm", "fused_add_rmsnorm", "rmsnorm_fp8", "fused_add_rmsnorm_fp8", "norm",
    "sum_add_rmsnorm",
    "silu_and_mul", "silu_and_mul_fp8",
    "fp8_gemm", "fp8_weight_preshuffle", "PreshuffledWeight", "fp8_gemm_workspace",
    "fp8_gemm_preshuffled_noalloc",
    "set_tile", "set_gemm_config", "set_gemm_splits", "last_plan", "norm_plan", "ArnError",
]

_DTYPES = {torch.bfloat16: _lib.BF16, torch.float16: _lib.FP16}
FP8_DTYPE = torch.float8_e4m3fn


def _rows(t: torch.Tensor, name: str):
    """(rows, hidden, row_stride) of a tensor viewed as 2-D rows, no copy."""
    return _lib.native().row_view(t, name)


def _dtype_code(x: torch.Tensor) -> int:
    try:
        return _DTYPES[x.dtype]
    except KeyError:
        raise ValueError(f"activations must be bfloat16 or float16, got {x.dtype}") from None


def _check_weight(weight, x, hidden):
    if weight is None:
        return None
    if weight.dtype != x.dtype:
        raise ValueError("weight dtype must match x dtype")
    if weight.dim() != 1 or weight.shape[0] != hidden or (hidden > 1 and weight.stride(0) != 1):
        raise ValueError(f"weight must be a contiguous vector of {hidden} elements")
    if weight.device != x.device:
        raise ValueError("weight must be on x's device")
    return weight.data_ptr()


def _check_device(x: torch.Tensor):
    if x.device.type != "cuda":
        raise ValueError("tensors must live on a GPU device")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_SAME_DEVICE = contextlib.nullcontext()


def _stream(x: torch.Tensor) -> int:
    """The current HIP stream of x's device (a raw handle)."""
    if _raw_stream is not None:
        return _raw_stream(x.device.index)
    return torch.cuda.current_stream(x.device).cuda_stream


def _on(x: torch.Tensor):
    """Make x's device current for the call (a no-op when it already is)."""
    idx = x.device.index
    return _SAME_DEVICE if idx == torch.cuda.current_device() else torch.cuda.device(idx)


def _out_like(x, out, dtype, name="out"):
    if out is None:
        return torch.empty(x.shape, dtype=dtype, device=x.device)
    if out.shape != x.shape or out.dtype != dtype or out.device != x.device:
        raise ValueError(f"{name} must have x's shape and dtype {dtype} on x's device")
    return out


def rmsnorm(x: torch.Tensor, weight: torch.Tensor | None, eps: float,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """out = x / sqrt(mean(x^2, -1) + eps) * weight  (arn_rmsnorm)."""
    return _lib.native().rmsnorm(x, weight, eps, out)


def fused_add_rmsnorm(x: torch.Tensor, residual: torch.Tensor, weight: torch.Tensor | None,
                      eps: float, out: torch.Tensor | None = None) -> torch.Tensor:
    """residual <- x + residual (rounded to the 16-bit type, in place);
    returns out = RMSNorm(residual)  (arn_fused_add_rmsnorm)."""
    return _lib.native().fused_add_rmsnorm(x, residual, weight, eps, out)


def _fp8_scale(x, rows, scale, dynamic, scales_out):
    if dynamic:
        if scales_out is None:
            scales_out = torch.empty(x.shape[:-1] if x.dim() > 1 else (1,),
                                     dtype=torch.float32, device=x.device)
        if (scales_out.dtype != torch.float32 or scales_out.numel() != rows
                or not scales_out.is_contiguous() or scales_out.device != x.device):
            raise ValueError(f"scales_out must be {rows} contiguous float32 values on x's device")
        return scales_out, _lib.FP8_DYNAMIC
    if scale is None:
        raise ValueError("static FP8 needs `scale` (one float32 dequant scale on the device)")
    if scale.dtype != torch.float32 or scale.numel() != 1 or scale.device != x.device:
        raise ValueError("scale must be one float32 value on x's device")
    return scale, _lib.FP8_STATIC


def rmsnorm_fp8(x: torch.Tensor, weight: torch.Tensor | None, eps: float,
                scale: torch.Tensor | None = None, dynamic: bool = False,
                out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None):
    """RMSNorm with an OCP e4m3 output  (arn_rmsnorm_fp8).

    Static (``scale`` given, dequant scale s): codes = e4m3(y / s).
    Dynamic: per-row scales = max|y| / 448 are written and returned.
    Returns (codes as float8_e4m3fn, scale tensor)."""
    return _lib.native().rmsnorm_fp8(x, weight, eps, scale, dynamic, out, scales_out)


def fused_add_rmsnorm_fp8(x: torch.Tensor, residual: torch.Tensor,
                          weight: torch.Tensor | None, eps: float,
                          scale: torch.Tensor | None = None, dynamic: bool = False,
                          out: torch.Tensor | None = None,
                          scales_out: torch.Tensor | None = None):
    """residual <- x + residual; codes = e4m3(RMSNorm(residual) / scale)
    (arn_fused_add_rmsnorm_fp8).  Returns (codes, scale tensor)."""
    return _lib.native().fused_add_rmsnorm_fp8(x, residual, weight, eps, scale, dynamic, out,
                                                scales_out)


def norm(x: torch.Tensor, weight: torch.Tensor | None, eps: float,
         residual: torch.Tensor | None = None, variance_size: int | None = None,
         fp8: str | None = None, scale: torch.Tensor | None = None,
         out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None):
    """Every norm form through arn_norm, with an optional variance-size
    override (mean of squares over the first ``variance_size`` channels).
    ``fp8``: None (16-bit out), "static" (needs ``scale``) or "dynamic".
    Returns out, or (codes, scale tensor) for FP8."""
    return _lib.native().norm(x, weight, eps, residual,
                              0 if variance_size is None else int(variance_size), fp8 or "",
                              scale, out, scales_out)


def sum_add_rmsnorm(parts, weight: torch.Tensor | None, eps: float,
                    residual: torch.Tensor | None = None, fp8: str | None = None,
                    scale: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    scales_out: torch.Tensor | None = None):
    """The all-reduce reduction fused with the residual add + RMSNorm
    (arn_sum_add_rmsnorm): x = the fp32 rank-order sum of the tensors in
    ``parts`` (1..8, same shape, dtype and row layout), rounded once to 16
    bits; then residual += x (when given) and out = norm(residual or x).
    ``fp8`` as in norm().  Returns out, or (codes, scale tensor) for FP8."""
    import ctypes

    parts = list(parts)
    if not 1 <= len(parts) <= 8:
        raise ValueError("parts must hold 1 to 8 tensors")
    x = parts[0]
    _check_device(x)
    dt = _dtype_code(x)
    rows, hidden, xs = _rows(x, "parts[0]")
    for i, p in enumerate(parts[1:], 1):
        if p.dtype != x.dtype or p.shape != x.shape or p.device != x.device:
            raise ValueError(f"parts[{i}] must match parts[0] in shape, dtype and device")
        if _rows(p, f"parts[{i}]")[2] != xs:
            raise ValueError(f"parts[{i}] must have the row stride of parts[0]")
    rs = 0
    if residual is not None:
        if residual.dtype != x.dtype or residual.shape != x.shape or residual.device != x.device:
            raise ValueError("residual must match the parts in shape, dtype and device")
        _, _, rs = _rows(residual, "residual")
    out = _out_like(x, out, FP8_DTYPE if fp8 else x.dtype)
    _, _, os_ = _rows(out, "out")
    wp = _check_weight(weight, x, hidden)
    sc = None
    fmt = _lib.OUT_16BIT
    if fp8:
        if fp8 not in ("static", "dynamic"):
            raise ValueError("fp8 must be None, 'static' or 'dynamic'")
        sc, _ = _fp8_scale(x, rows, scale, fp8 == "dynamic", scales_out)
        fmt = _lib.OUT_FP8_DYNAMIC if fp8 == "dynamic" else _lib.OUT_FP8_STATIC
    ptrs = (ctypes.c_void_p * len(parts))(*[p.data_ptr() for p in parts])
    args = _lib.SumNormArgs(
        struct_size=ctypes.sizeof(_lib.SumNormArgs), dtype=dt, out_format=fmt,
        out=out.data_ptr(), out_stride=os_, scale=sc.data_ptr() if sc is not None else None,
        parts=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), nparts=len(parts),
        parts_stride=xs, residual=residual.data_ptr() if residual is not None else None,
        residual_stride=rs, weight=wp, eps=float(eps), rows=rows, hidden=hidden,
        stream=_stream(x))
    lib = _lib.load()
    with _on(x):
        st = lib.arn_sum_add_rmsnorm(ctypes.byref(args))
    _lib.check(st, "arn_sum_add_rmsnorm")
    return (out, sc) if fp8 else out


def silu_and_mul(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out = silu(x[..., :d]) * x[..., d:] for x of shape [..., 2d]
    (arn_silu_and_mul with gate = x, up = x + d)."""
    return _lib.native().silu_and_mul(x, out)


def silu_and_mul_fp8(x: torch.Tensor, scale: torch.Tensor | None = None, dynamic: bool = False,
                     out: torch.Tensor | None = None, scales_out: torch.Tensor | None = None):
    """SwiGLU of a [..., 2d] gate|up tensor with an OCP e4m3 output
    (arn_silu_and_mul_fp8).  Returns (codes, scale tensor)."""
    return _lib.native().silu_and_mul_fp8(x, scale, dynamic, out, scales_out)


class PreshuffledWeight:
    """An e4m3 weight [N, K] in the GEMM's pre-shuffled tile order
    (arn_fp8_weight_preshuffle); pass it to fp8_gemm in place of the
    row-major weight."""

    def __init__(self, data: torch.Tensor, n: int, k: int):
        self.data = data  # uint8, arn_fp8_weight_preshuffled_bytes(n, k) bytes
        self.n = n
        self.k = k
        self.device = data.device

    @property
    def shape(self):
        return (self.n, self.k)


def fp8_weight_preshuffle(b: torch.Tensor) -> PreshuffledWeight:
    """The pre-shuffled copy of an e4m3 weight b [N, K] (out-feature major)."""
    _check_device(b)
    if b.dtype not in (FP8_DTYPE, torch.uint8) or b.dim() != 2 or b.stride(1) != 1:
        raise ValueError("b must be a 2-D e4m3 (or uint8) tensor with unit column stride")
    n, k = b.shape
    lib = _lib.load()
    size = lib.arn_fp8_weight_preshuffled_bytes(n, k)
    if size < 0:
        raise ValueError("b must have K >= 1")
    dst = torch.empty(max(size, 16), dtype=torch.uint8, device=b.device)
    with _on(b):
        st = lib.arn_fp8_weight_preshuffle(dst.data_ptr(), b.data_ptr(), b.stride(0), n, k,
                                           _stream(b))
    _lib.check(st, "arn_fp8_weight_preshuffle")
    return PreshuffledWeight(dst, n, k)


def fp8_gemm_workspace(m: int, n: int, k: int, device="cuda") -> torch.Tensor:
    """A zero-filled split-K workspace for GEMMs of up to m x n outputs
    (arn_fp8_gemm_workspace_bytes); reusable by later calls on one stream."""
    size = _lib.load().arn_fp8_gemm_workspace_bytes(m, n, k)
    if size < 0:
        raise ValueError("invalid GEMM shape")
    return torch.zeros(size, dtype=torch.uint8, device=device)


def fp8_gemm(a: torch.Tensor, scale_a: torch.Tensor, b, scale_b: torch.Tensor,
             out_dtype: torch.dtype = torch.bfloat16,
             out: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """out[i, j] = scale_a(i) * scale_b(j) * sum_t a[i, t] * b[j, t]
    (arn_fp8_gemm) for e4m3 codes a [M, K] (float8_e4m3fn or uint8) and b
    [N, K] (the weight, out-feature major) or its PreshuffledWeight
    (arn_fp8_gemm_preshuffled); scale_a holds M or 1 float32 values,
    scale_b N or 1.  With a workspace (fp8_gemm_workspace) K may also be
    split across blocks (the _ws entry points)."""
    if isinstance(b, PreshuffledWeight):
        bt, pre_n, pre_k = b.data, b.n, b.k
    else:
        bt, pre_n, pre_k = b, -1, -1
    return _lib.native().fp8_gemm(a, scale_a, bt, scale_b, _DTYPES.get(out_dtype, -1), out,
                                  workspace, pre_n, pre_k)


def fp8_gemm_preshuffled_noalloc(a: torch.Tensor, scale_a: torch.Tensor, b: "PreshuffledWeight",
                                 scale_b: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                                 out: torch.Tensor | None = None) -> torch.Tensor:
    """fp8_gemm with a pre-shuffled weight and K split across blocks as with a
    workspace, the partial tiles held in the library's own device array
    (arn_fp8_gemm_preshuffled_noalloc): no device memory is allocated when
    `out` is given.  Calls on one GPU must not overlap."""
    if not isinstance(b, PreshuffledWeight):
        raise ValueError("b must be a PreshuffledWeight")
    return _lib.native().fp8_gemm_preshuffled_noalloc(a, scale_a, b.data, b.n, b.k, scale_b,
                                                      _DTYPES.get(out_dtype, -1), out)


def set_tile(waves_per_row: int = 0, vec_per_lane: int = 0) -> None:
    """Force a kernel shape for this thread's later calls ((0, 0) = automatic;
    other threads are not affected)."""
    _lib.check(_lib.load().arn_set_tile(waves_per_row, vec_per_lane), "arn_set_tile")


def set_gemm_config(col_tiles: int = 0, waves: int = 0) -> None:
    """Force the e4m3 GEMM's block shape for this thread's later calls
    ((0, 0) = automatic; other threads are not affected)."""
    _lib.check(_lib.load().arn_set_gemm_config(col_tiles, waves), "arn_set_gemm_config")


def set_gemm_splits(splits: int = 0) -> None:
    """Force the number of K splits of this thread's later workspace GEMM
    calls (0 = automatic; other threads are not affected)."""
    _lib.check(_lib.load().arn_set_gemm_splits(splits), "arn_set_gemm_splits")


def norm_plan(dtype: str, rows: int, hidden: int, *, fused: bool = False, fp8: str | None = None,
              stride: int | None = None, variance_size: int = 0, weight: bool = True,
              compute_units: int = 256, align: int = 16) -> str:
    """The kernel arn_norm would launch for rows of `hidden` elements (row
    stride `stride`, every base aligned to `align` bytes) on a device with
    `compute_units` CUs, from arn_norm_plan: nothing is launched and no
    memory is touched (the pointers passed are stand-in addresses).
    Returns arn_last_plan's description, "" for rows == 0; raises ArnError
    for a call arn_norm would refuse."""
    import ctypes

    if dtype not in ("bf16", "fp16"):
        raise ValueError("dtype must be 'bf16' or 'fp16'")
    stride = hidden if stride is None else stride
    base = 1 << 40  # stand-in device addresses, far apart, `align`-aligned
    fmt = {None: _lib.OUT_16BIT, "static": _lib.OUT_FP8_STATIC,
           "dynamic": _lib.OUT_FP8_DYNAMIC}[fp8]
    args = _lib.NormArgs(
        struct_size=ctypes.sizeof(_lib.NormArgs), dtype=_lib.BF16 if dtype == "bf16" else _lib.FP16,
        out_format=fmt, out=base + 4 * align, out_stride=stride,
        scale=base + (1 << 36) if fp8 else None, x=base + (2 << 36) + align, x_stride=stride,
        residual=base + (3 << 36) + 2 * align if fused else None, residual_stride=stride,
        weight=base + (4 << 36) + 3 * align if weight else None, eps=1e-6, rows=rows,
        hidden=hidden, variance_size=variance_size, stream=None)
    buf = ctypes.create_string_buffer(160)
    st = _lib.load().arn_norm_plan(ctypes.byref(args), compute_units, buf, len(buf))
    _lib.check(st, "arn_norm_plan")
    return buf.value.decode()


def last_plan() -> str:
    """The kernel shape of this thread's last launch."""
    import ctypes

    buf = ctypes.create_string_buffer(160)
    _lib.load().arn_last_plan(buf, len(buf))
    return buf.value.decode()
