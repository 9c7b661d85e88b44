"""Loaders for libarn.so (the C ABI in include/arn.h, through ctypes) and for
the extension module lib/_native, which marshals the binding's per-call
arguments in C++ and calls the same library.

torch is imported first: it ships its own HIP runtime, and loading libarn.so
afterwards makes the library's libamdhip64.so.7 dependency resolve to that
same, already loaded runtime, so torch's streams and device pointers are
valid in the library.
"""
from __future__ import annotations

import ctypes
import importlib.util
import os
import threading

import torch  # noqa: F401  (must precede the library load; see above)

from . import build as _build

LIB_PATH = _build.LIB_PATH

OK, EINVAL, EUNSUPPORTED, ELAUNCH = 0, 1, 2, 3
BF16, FP16 = 0, 1
FP8_STATIC, FP8_DYNAMIC = 0, 1

# Every function include/arn.h and include/arn_tuning.h declare, with its
# ctypes signature.
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
SIGNATURES = {
    "arn_rmsnorm": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, ctypes.c_float, _i64, _i64,
                                   ctypes.c_int, _vp]),
    "arn_fused_add_rmsnorm": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _vp,
                                             ctypes.c_float, _i64, _i64, ctypes.c_int, _vp]),
    "arn_rmsnorm_fp8": (ctypes.c_int, [_vp, _i64, _vp, ctypes.c_int, _vp, _i64, _vp,
                                       ctypes.c_float, _i64, _i64, ctypes.c_int, _vp]),
    "arn_fused_add_rmsnorm_fp8": (ctypes.c_int, [_vp, _i64, _vp, ctypes.c_int, _vp, _i64, _vp,
                                                 _i64, _vp, ctypes.c_float, _i64, _i64,
                                                 ctypes.c_int, _vp]),
    "arn_silu_and_mul": (ctypes.c_int, [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                        ctypes.c_int, _vp]),
    "arn_silu_and_mul_fp8": (ctypes.c_int, [_vp, _i64, _vp, ctypes.c_int, _vp, _i64, _vp, _i64,
                                            _i64, _i64, ctypes.c_int, _vp]),
    "arn_norm": (ctypes.c_int, [_vp]),
    "arn_sum_add_rmsnorm": (ctypes.c_int, [_vp]),
    "arn_fp8_gemm": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _i64, _vp, ctypes.c_int, _vp,
                                    _i64, _vp, ctypes.c_int, _i64, _i64, _i64, _vp]),
    "arn_fp8_weight_preshuffled_bytes": (_i64, [_i64, _i64]),
    "arn_fp8_weight_preshuffle": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _vp]),
    "arn_fp8_gemm_preshuffled": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _i64, _vp,
                                                ctypes.c_int, _vp, _vp, ctypes.c_int, _i64, _i64,
                                                _i64, _vp]),
    "arn_fp8_gemm_workspace_bytes": (_i64, [_i64, _i64, _i64]),
    "arn_fp8_gemm_ws": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _i64, _vp, ctypes.c_int, _vp,
                                       _i64, _vp, ctypes.c_int, _i64, _i64, _i64, _vp,
                                       ctypes.c_size_t, _vp]),
    "arn_fp8_gemm_preshuffled_ws": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _i64, _vp,
                                                   ctypes.c_int, _vp, _vp, ctypes.c_int, _i64,
                                                   _i64, _i64, _vp, ctypes.c_size_t, _vp]),
    "arn_fp8_gemm_preshuffled_noalloc": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _i64, _vp,
                                                        ctypes.c_int, _vp, _vp, ctypes.c_int,
                                                        _i64, _i64, _i64, _vp]),
    "arn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "arn_abi_version": (ctypes.c_int, []),
    "arn_set_tile": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "arn_set_gemm_config": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
    "arn_set_gemm_splits": (ctypes.c_int, [ctypes.c_int]),
    "arn_last_plan": (ctypes.c_int, [ctypes.c_char_p, ctypes.c_size_t]),
    "arn_norm_plan": (ctypes.c_int, [_vp, ctypes.c_int, ctypes.c_char_p, ctypes.c_size_t]),
}

ABI_VERSION = 6

OUT_16BIT, OUT_FP8_STATIC, OUT_FP8_DYNAMIC = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 8 << 20


class NormArgs(ctypes.Structure):
    """struct arn_norm_args of include/arn.h."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("dtype", ctypes.c_int),
        ("out_format", ctypes.c_int),
        ("out", ctypes.c_void_p),
        ("out_stride", ctypes.c_int64),
        ("scale", ctypes.c_void_p),
        ("x", ctypes.c_void_p),
        ("x_stride", ctypes.c_int64),
        ("residual", ctypes.c_void_p),
        ("residual_stride", ctypes.c_int64),
        ("weight", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("rows", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("variance_size", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
    ]


class SumNormArgs(ctypes.Structure):
    """struct arn_sum_norm_args of include/arn.h."""
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("dtype", ctypes.c_int),
        ("out_format", ctypes.c_int),
        ("out", ctypes.c_void_p),
        ("out_stride", ctypes.c_int64),
        ("scale", ctypes.c_void_p),
        ("parts", ctypes.POINTER(ctypes.c_void_p)),
        ("nparts", ctypes.c_int),
        ("parts_stride", ctypes.c_int64),
        ("residual", ctypes.c_void_p),
        ("residual_stride", ctypes.c_int64),
        ("weight", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("rows", ctypes.c_int64),
        ("hidden", ctypes.c_int64),
        ("stream", ctypes.c_void_p),
    ]


class ArnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libarn.so, building it first only if it is not there at all."""
    global _lib
    if _lib is not None:  # loaded: no lock on the per-call path
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path) and path == LIB_PATH:
            _build.build()
        if not os.path.exists(path):
            raise ImportError(f"libarn.so not found at {path}; run "
                              "`python -m residual_add_rmsnorm_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.arn_abi_version() != ABI_VERSION:
            raise ImportError(f"libarn.so ABI {lib.arn_abi_version()} != {ABI_VERSION}")
        _lib = lib
        return lib


# The entry points the extension module calls, bound to the addresses of
# this ctypes handle so that both reach one copy of the library.
NATIVE_ENTRY_POINTS = (
    "arn_rmsnorm", "arn_fused_add_rmsnorm", "arn_rmsnorm_fp8", "arn_fused_add_rmsnorm_fp8",
    "arn_norm", "arn_silu_and_mul", "arn_silu_and_mul_fp8", "arn_fp8_gemm", "arn_fp8_gemm_ws",
    "arn_fp8_gemm_preshuffled", "arn_fp8_gemm_preshuffled_ws", "arn_fp8_gemm_preshuffled_noalloc",
    "arn_fp8_weight_preshuffled_bytes", "arn_status_str",
)

_native = None


def native(path: str | None = None):
    """The extension module (lib/_native), bound to libarn.so; built first
    only if it is not there at all."""
    global _native
    if _native is not None:
        return _native
    with _lock:
        if _native is not None:
            return _native
        path = path or _build.NATIVE_PATH
        if not os.path.exists(path) and path == _build.NATIVE_PATH:
            _build.build_native()
        if not os.path.exists(path):
            raise ImportError(f"the binding's extension module is not at {path}; run "
                              "`python -m residual_add_rmsnorm_amd.build`")
    lib = load()
    with _lock:
        if _native is None:
            spec = importlib.util.spec_from_file_location("residual_add_rmsnorm_amd._native", path)
            mod = importlib.util.module_from_spec(spec)
            spec.loader.exec_module(mod)
            mod.bind({name: ctypes.cast(getattr(lib, name), ctypes.c_void_p).value
                      for name in NATIVE_ENTRY_POINTS}, check)
            _native = mod
    return _native


def status_str(status: int) -> str:
    return load().arn_status_str(status).decode()


def check(status: int, what: str) -> None:
    if status != OK:
        raise ArnError(status, what)
