"""Plain fp64 CPU oracle for residual-add + RMSNorm (+ OCP e4m3).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The
product library never loads it, and it shares no code with the HIP path.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one step per
function, each citing the passage it follows).  This module only compiles it
with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_HDR = os.path.join(_HERE, "oracle.h")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP16 = 1
FP8_NONE = -1
FP8_STATIC = 0
FP8_DYNAMIC = 1

DTYPES = {"bf16": BF16, "fp16": FP16}

# ISO C, no contraction of a*b+c into fma, no fast-math: every double
# operation in oracle.c is rounded exactly as written.
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lock = threading.Lock()
_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile oracle.c into a shared library with gcc."""
    cmd = ["gcc", *GCC_FLAGS, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _stale(lib_path: str) -> bool:
    if not os.path.exists(lib_path):
        return True
    t = os.path.getmtime(lib_path)
    return any(os.path.getmtime(p) > t for p in (_SRC, _HDR))


def bind(lib_path: str) -> ctypes.CDLL:
    """Load a compiled oracle and declare its C signatures."""
    lib = ctypes.CDLL(lib_path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.orc_decode16.argtypes = [ctypes.c_int, ctypes.c_uint16]
    lib.orc_decode16.restype = ctypes.c_double
    lib.orc_encode16.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.orc_encode16.restype = ctypes.c_uint16
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_add_rmsnorm.argtypes = [
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        u16p, ctypes.c_int64,
        u16p, ctypes.c_int64,
        u16p, ctypes.c_float,
        u16p, ctypes.POINTER(ctypes.c_double), u16p,
        ctypes.c_int, ctypes.c_float,
        ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_float),
    ]
    lib.orc_add_rmsnorm.restype = ctypes.c_int
    lib.orc_add_rmsnorm_var.argtypes = (lib.orc_add_rmsnorm.argtypes[:3] + [ctypes.c_int64]
                                        + lib.orc_add_rmsnorm.argtypes[3:])
    lib.orc_add_rmsnorm_var.restype = ctypes.c_int
    lib.orc_residual16.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint16),
                                   ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_uint16)]
    lib.orc_residual16.restype = ctypes.c_int
    lib.orc_sum_parts16.argtypes = [ctypes.c_int, ctypes.c_int,
                                    ctypes.POINTER(ctypes.POINTER(ctypes.c_uint16)),
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.POINTER(ctypes.c_uint16)]
    lib.orc_sum_parts16.restype = ctypes.c_int
    lib.orc_silu.argtypes = [ctypes.c_double]
    lib.orc_silu.restype = ctypes.c_double
    lib.orc_silu_and_mul.argtypes = [
        ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
        u16p, ctypes.c_int64, u16p, ctypes.c_int64,
        ctypes.POINTER(ctypes.c_double), u16p,
        ctypes.c_int, ctypes.c_float,
        ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_float),
    ]
    lib.orc_silu_and_mul.restype = ctypes.c_int
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.orc_fp8_gemm.argtypes = [
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        u8p, ctypes.c_int64, f32p, ctypes.c_int,
        u8p, ctypes.c_int64, f32p, ctypes.c_int,
        ctypes.c_int, f64p, u16p,
    ]
    lib.orc_fp8_gemm.restype = ctypes.c_int
    return lib


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if _stale(LIB_PATH):
                build()
            _lib = bind(LIB_PATH)
        return _lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """numpy front end over one compiled oracle library."""

    def __init__(self, cdll: ctypes.CDLL | None = None):
        self.c = cdll if cdll is not None else lib()

    # -- scalar codecs ---------------------------------------------------
    def decode16(self, dtype: int, bits: int) -> float:
        return self.c.orc_decode16(dtype, bits)

    def encode16(self, dtype: int, v: float) -> int:
        return self.c.orc_encode16(dtype, v)

    def e4m3_decode(self, code: int) -> float:
        return self.c.orc_e4m3_decode(code)

    def e4m3_encode(self, v: float) -> int:
        return self.c.orc_e4m3_encode(v)

    # -- the operator ------------------------------------------------------
    def add_rmsnorm(self, dtype, x, residual, weight, eps, hidden=None,
                    fp8_mode=FP8_NONE, static_scale=0.0, want_y=True, variance_size=None):
        """Run the reference on 2-D uint16 arrays (row stride = shape[1]).

        ``hidden`` defaults to the full row; a smaller value leaves the
        columns beyond it (row padding) out of the computation.
        ``variance_size`` (default ``hidden``) limits the mean of squares to
        the first that many channels.
        Returns a dict with r16, y (float64), y16, and q / scales for FP8.
        """
        if isinstance(dtype, str):
            dtype = DTYPES[dtype]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        rows, stride = x.shape
        hidden = stride if hidden is None else int(hidden)
        if residual is not None:
            residual = np.ascontiguousarray(residual, dtype=np.uint16)
            assert residual.shape[0] == rows
        if weight is not None:
            weight = np.ascontiguousarray(weight, dtype=np.uint16)
            assert weight.shape[0] >= hidden
        r16 = np.empty((rows, hidden), np.uint16)
        y = np.empty((rows, hidden), np.float64) if want_y else None
        y16 = np.empty((rows, hidden), np.uint16)
        q = np.empty((rows, hidden), np.uint8) if fp8_mode != FP8_NONE else None
        scales = np.empty((rows,), np.float32) if fp8_mode == FP8_DYNAMIC else None
        rc = self.c.orc_add_rmsnorm_var(
            dtype, rows, hidden, hidden if variance_size is None else int(variance_size),
            _ptr(x, ctypes.c_uint16), stride,
            _ptr(residual, ctypes.c_uint16),
            residual.shape[1] if residual is not None else 0,
            _ptr(weight, ctypes.c_uint16), float(eps),
            _ptr(r16, ctypes.c_uint16), _ptr(y, ctypes.c_double),
            _ptr(y16, ctypes.c_uint16),
            fp8_mode, float(static_scale),
            _ptr(q, ctypes.c_uint8), _ptr(scales, ctypes.c_float),
        )
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        out = {"r16": r16, "y16": y16}
        if want_y:
            out["y"] = y
        if q is not None:
            out["q"] = q
        if scales is not None:
            out["scales"] = scales
        return out

    def residual16(self, dtype, x, res):
        """The stored residual of each pair (x[i], res[i]) of two 1-D uint16
        arrays of equal length."""
        if isinstance(dtype, str):
            dtype = DTYPES[dtype]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        res = np.ascontiguousarray(res, dtype=np.uint16)
        assert x.shape == res.shape and x.ndim == 1
        out = np.empty_like(x)
        rc = self.c.orc_residual16(dtype, x.size, _ptr(x, ctypes.c_uint16),
                                   _ptr(res, ctypes.c_uint16), _ptr(out, ctypes.c_uint16))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out

    def sum_parts(self, dtype, parts, hidden=None):
        """The all-reduce reduction of a list of 2-D uint16 arrays of equal
        shape (row stride = shape[1]): fp32 accumulation in list order, one
        rounding.  Returns rows x hidden uint16 patterns."""
        if isinstance(dtype, str):
            dtype = DTYPES[dtype]
        parts = [np.ascontiguousarray(p, dtype=np.uint16) for p in parts]
        rows, stride = parts[0].shape
        assert all(p.shape == (rows, stride) for p in parts)
        hidden = stride if hidden is None else int(hidden)
        out = np.empty((rows, hidden), np.uint16)
        arr = (ctypes.POINTER(ctypes.c_uint16) * len(parts))(
            *[_ptr(p, ctypes.c_uint16) for p in parts])
        rc = self.c.orc_sum_parts16(dtype, len(parts), arr, stride, rows, hidden,
                                    _ptr(out, ctypes.c_uint16))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return out

    def sum_add_rmsnorm(self, dtype, parts, residual, weight, eps, hidden=None, **kw):
        """All-reduce of the parts, then the (fused) add + RMSNorm on the
        reduced rows: the unfused definition of the fused kernel."""
        x16 = self.sum_parts(dtype, parts, hidden)
        res = None if residual is None else np.ascontiguousarray(residual)[:, :x16.shape[1]]
        return self.add_rmsnorm(dtype, x16, res, weight, eps, **kw)

    def silu(self, g: float) -> float:
        return self.c.orc_silu(g)

    def silu_and_mul(self, dtype, x, d=None, fp8_mode=FP8_NONE, static_scale=0.0, want_y=True):
        """SwiGLU on a 2-D uint16 array whose row holds the gate in columns
        [0, d) and up in [d, 2d) (row stride = shape[1]; d defaults to half
        of it).  Returns a dict with y (float64), y16, and q / scales."""
        if isinstance(dtype, str):
            dtype = DTYPES[dtype]
        x = np.ascontiguousarray(x, dtype=np.uint16)
        rows, stride = x.shape
        d = stride // 2 if d is None else int(d)
        assert 2 * d <= stride
        self._keep = x
        base = x.ctypes.data
        gate = ctypes.cast(base, ctypes.POINTER(ctypes.c_uint16))
        up = ctypes.cast(base + 2 * d, ctypes.POINTER(ctypes.c_uint16))
        return self._silu_and_mul(dtype, rows, d, gate, stride, up, stride, fp8_mode,
                                  static_scale, want_y)

    def silu_and_mul_split(self, dtype, gate, up, d=None, fp8_mode=FP8_NONE, static_scale=0.0):
        """SwiGLU with the gate and up halves in two separate 2-D arrays,
        each with its own row stride (shape[1])."""
        if isinstance(dtype, str):
            dtype = DTYPES[dtype]
        gate = np.ascontiguousarray(gate, dtype=np.uint16)
        up = np.ascontiguousarray(up, dtype=np.uint16)
        assert gate.shape[0] == up.shape[0]
        d = min(gate.shape[1], up.shape[1]) if d is None else int(d)
        self._keep = (gate, up)
        return self._silu_and_mul(dtype, gate.shape[0], d, _ptr(gate, ctypes.c_uint16),
                                  gate.shape[1], _ptr(up, ctypes.c_uint16), up.shape[1],
                                  fp8_mode, static_scale, True)

    def _silu_and_mul(self, dtype, rows, d, gate, gate_stride, up, up_stride, fp8_mode,
                      static_scale, want_y):
        y = np.empty((rows, d), np.float64) if want_y else None
        y16 = np.empty((rows, d), np.uint16)
        q = np.empty((rows, d), np.uint8) if fp8_mode != FP8_NONE else None
        scales = np.empty((rows,), np.float32) if fp8_mode == FP8_DYNAMIC else None
        rc = self.c.orc_silu_and_mul(dtype, rows, d, gate, gate_stride, up, up_stride,
                                     _ptr(y, ctypes.c_double), _ptr(y16, ctypes.c_uint16),
                                     fp8_mode, float(static_scale),
                                     _ptr(q, ctypes.c_uint8), _ptr(scales, ctypes.c_float))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        out = {"y16": y16}
        if want_y:
            out["y"] = y
        if q is not None:
            out["q"] = q
        if scales is not None:
            out["scales"] = scales
        return out


    def fp8_gemm(self, a, sa, b, sb, k=None, out_dtype="bf16"):
        """C = diag(sa) dec(A) dec(B)^T diag(sb) for uint8 code arrays
        A (M x lda) and B (N x ldb); sa / sb hold M / N per-row scales or one
        per-tensor scale.  Returns dict c (float64) and c16."""
        a = np.ascontiguousarray(a, dtype=np.uint8)
        b = np.ascontiguousarray(b, dtype=np.uint8)
        sa = np.ascontiguousarray(np.atleast_1d(sa), dtype=np.float32)
        sb = np.ascontiguousarray(np.atleast_1d(sb), dtype=np.float32)
        m, lda = a.shape
        n, ldb = b.shape
        k = min(lda, ldb) if k is None else int(k)
        c = np.empty((m, n), np.float64)
        c16 = np.empty((m, n), np.uint16)
        rc = self.c.orc_fp8_gemm(m, n, k, _ptr(a, ctypes.c_uint8), lda, _ptr(sa, ctypes.c_float),
                                 int(sa.size > 1),
                                 _ptr(b, ctypes.c_uint8), ldb, _ptr(sb, ctypes.c_float),
                                 int(sb.size > 1), DTYPES[out_dtype],
                                 _ptr(c, ctypes.c_double), _ptr(c16, ctypes.c_uint16))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return {"c": c, "c16": c16}


def oracle() -> Oracle:
    return Oracle()
