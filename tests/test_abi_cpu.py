"""The C ABI without a GPU: the library loads, exports every function
include/arn.h declares, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest
import torch
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

from residual_add_rmsnorm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arn.h")
TUNING_HEADER = os.path.join(ROOT, "include", "arn_tuning.h")


PROBE_HEADER = os.path.join(ROOT, "include", "arn_probe.h")


def header_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(arn_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_bound_functions():
    product, tuning = header_functions(), header_functions(TUNING_HEADER)
    assert not set(product) & set(tuning)
    assert sorted(product + tuning) == sorted(_lib.SIGNATURES)
    # the product header declares nothing that sets state
    assert not any(n.startswith("arn_set_") for n in product)
    assert tuning == ["arn_last_plan", "arn_norm_plan", "arn_set_gemm_config",
                      "arn_set_gemm_splits", "arn_set_tile"]


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (arn_\w+)", out))
    for name in header_functions() + header_functions(TUNING_HEADER):
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert lib.arn_abi_version() == _lib.ABI_VERSION == 6


def test_probe_library_exports_its_header():
    """The streaming probe the benchmark measures ceilings with lives in its
    own library and exports what include/arn_probe.h declares."""
    from residual_add_rmsnorm_amd import build

    out = subprocess.run(["nm", "-D", "--defined-only", build.PROBE_LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (arn_\w+)", out))
    assert header_functions(PROBE_HEADER) == ["arn_probe_empty", "arn_probe_rows",
                                              "arn_probe_stream", "arn_probe_stream_many"]
    assert set(header_functions(PROBE_HEADER)) <= exported
    probe = ctypes.CDLL(build.PROBE_LIB_PATH)
    f = probe.arn_probe_stream
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 4 + [ctypes.c_int64, ctypes.c_int,
                                                               ctypes.c_int, ctypes.c_void_p]
    # argument errors are caught before any HIP call
    assert f(1, 1, 0, 16, 16, 16, 16, 0, 1, 256, None) == 1        # n = 0
    assert f(1, 1, 0, 16, 16, 16, 16, 64, 1, 300, None) == 1       # block size
    assert f(2, 2, 0, 16, 16, 16, None, 64, 1, 256, None) == 1     # d missing
    assert f(2, 0, 0, 16, 16, 16, 16, 64, 1, 256, None) == 2       # mix not served
    e = probe.arn_probe_empty
    e.restype = ctypes.c_int
    e.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert e(0, 64, None) == 1 and e(1, 2048, None) == 1
    r = probe.arn_probe_rows
    r.restype = ctypes.c_int
    r.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [
        ctypes.c_void_p]
    assert r(0, 1, 16, 16, 16, 4, 16384 + 16, 16400, None) == 1   # row over 16 KiB
    assert r(0, 1, 16, 16, 16, 4, 100, 128, None) == 1            # not a multiple of 16
    assert r(4, 1, 16, 16, 16, 4, 128, 128, None) == 1            # mode
    assert r(0, 1, 16, 16, 16, 4, 128, 64, None) == 1             # pitch below the row
    assert r(0, 3, 16, 16, 16, 4, 128, 128, None) == 2            # rows per block


def test_hip_imports_resolve_in_torch_runtime():
    """libarn.so is loaded into processes whose HIP runtime is torch's
    bundled libamdhip64; every HIP symbol it imports must exist there."""
    imports = subprocess.run(["nm", "-D", "--undefined-only", _lib.LIB_PATH],
                             capture_output=True, text=True, check=True).stdout
    need = set(re.findall(r"U (_*hip\w+)@", imports))
    assert "hipLaunchKernel" in need
    torch_hip = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    have = subprocess.run(["nm", "-D", "--defined-only", torch_hip],
                          capture_output=True, text=True, check=True).stdout
    have = set(re.findall(r" T (_*hip\w+)@", have))
    assert need <= have, need - have


def test_status_strings(lib):
    assert lib.arn_status_str(0) == b"ok"
    assert lib.arn_status_str(1) == b"invalid argument"
    assert lib.arn_status_str(2) == b"unsupported shape or layout"
    assert lib.arn_status_str(3) == b"kernel launch failed"
    assert lib.arn_status_str(99) == b"unknown status"


# Fake, never dereferenced device addresses: validation must fail first.
P = 0x7F0000000000
Q = 0x7F0000100000
R = 0x7F0000200000
S = 0x7F0000300000


def _plain(lib, out=P, os_=64, x=Q, xs=64, w=None, eps=1e-6, rows=4, hidden=64, dt=0):
    return lib.arn_rmsnorm(out, os_, x, xs, w, eps, rows, hidden, dt, None)


def _fused(lib, out=P, os_=64, x=Q, xs=64, res=R, rs=64, w=None, eps=1e-6, rows=4, hidden=64,
           dt=0):
    return lib.arn_fused_add_rmsnorm(out, os_, x, xs, res, rs, w, eps, rows, hidden, dt, None)


def _fp8(lib, fused, out=P, os_=64, scale=S, mode=0, x=Q, xs=64, res=R, rs=64, w=None, eps=1e-6,
         rows=4, hidden=64, dt=0):
    if fused:
        return lib.arn_fused_add_rmsnorm_fp8(out, os_, scale, mode, x, xs, res, rs, w, eps, rows,
                                             hidden, dt, None)
    return lib.arn_rmsnorm_fp8(out, os_, scale, mode, x, xs, w, eps, rows, hidden, dt, None)


@pytest.mark.parametrize("case", [
    dict(dt=2), dict(dt=-1), dict(rows=-1), dict(hidden=0), dict(hidden=-5),
    dict(xs=63), dict(os_=32), dict(eps=-1e-6), dict(eps=float("nan")), dict(eps=float("inf")),
    dict(out=None), dict(x=None), dict(x=Q + 1), dict(out=P + 1), dict(w=S + 1),
    dict(out=Q, os_=128, xs=64),
])
def test_rmsnorm_rejects(lib, case):
    assert _plain(lib, **case) == _lib.EINVAL


@pytest.mark.parametrize("case", [
    dict(res=None), dict(rs=10), dict(res=Q), dict(res=P), dict(res=R + 1),
])
def test_fused_rejects(lib, case):
    assert _fused(lib, **case) == _lib.EINVAL


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("case", [
    dict(mode=2), dict(mode=-1), dict(scale=None), dict(scale=S + 2), dict(out=Q),
    dict(dt=5), dict(os_=3),
])
def test_fp8_rejects(lib, fused, case):
    assert _fp8(lib, fused, **case) == _lib.EINVAL


# Invalid arguments drawn in combination: any set of them is refused with
# ARN_EINVAL (before any HIP call: there is no GPU here, so a call that got
# past validation would report a launch failure instead).
VIOLATIONS = {
    "dtype": dict(dt=2), "rows": dict(rows=-3), "hidden": dict(hidden=0),
    "x_stride": dict(xs=63), "out_stride": dict(os_=32), "eps_negative": dict(eps=-1.0),
    "eps_nan": dict(eps=float("nan")), "eps_inf": dict(eps=float("inf")),
    "out_null": dict(out=None), "x_null": dict(x=None), "x_misaligned": dict(x=Q + 1),
    "w_misaligned": dict(w=S + 1), "scale_null": dict(scale=None),
    "scale_misaligned": dict(scale=S + 2), "mode": dict(mode=7),
    "res_null": dict(res=None), "res_stride": dict(rs=10), "res_is_x": dict(res=Q),
    "res_is_out": dict(res=P), "res_misaligned": dict(res=R + 1),
}


@settings(max_examples=300, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(names=st.lists(st.sampled_from(sorted(VIOLATIONS)), min_size=1, max_size=6, unique=True),
       fused=st.booleans())
def test_any_combination_of_invalid_arguments_is_refused(names, fused):
    lib = _lib.load()
    if not fused:
        names = [n for n in names if not n.startswith("res_")]
    assume(names)
    kw = {}
    for n in names:
        kw.update(VIOLATIONS[n])
    assert _fp8(lib, fused, **kw) == _lib.EINVAL, names


def test_zero_rows_is_a_no_op(lib):
    # no pointer is looked at and nothing is launched
    assert _plain(lib, out=None, x=None, rows=0) == _lib.OK
    assert _fused(lib, out=None, x=None, res=None, rows=0) == _lib.OK
    assert _fp8(lib, True, out=None, x=None, res=None, scale=None, rows=0) == _lib.OK


def test_set_tile(lib):
    assert lib.arn_set_tile(3, 3) == _lib.EINVAL
    assert lib.arn_set_tile(1, 16) == _lib.OK
    assert lib.arn_set_tile(16, 8) == _lib.OK
    assert lib.arn_set_tile(0, 0) == _lib.OK


def _norm_args(**kw):
    a = _lib.NormArgs(struct_size=ctypes.sizeof(_lib.NormArgs), dtype=0, out_format=0, out=P,
                      out_stride=64, scale=None, x=Q, x_stride=64, residual=R, residual_stride=64,
                      weight=None, eps=1e-6, rows=4, hidden=64, variance_size=0, stream=None)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("case", [
    dict(struct_size=8), dict(out_format=3), dict(variance_size=-1), dict(variance_size=65),
    dict(out_format=1, scale=None), dict(dtype=4), dict(residual=Q),
])
def test_norm_descriptor_rejects(lib, case):
    a = _norm_args(**case)
    assert lib.arn_norm(ctypes.byref(a)) == _lib.EINVAL
    assert lib.arn_norm(None) == _lib.EINVAL


def test_norm_descriptor_zero_rows(lib):
    a = _norm_args(rows=0, out=None, x=None, residual=None, variance_size=10)
    assert lib.arn_norm(ctypes.byref(a)) == _lib.OK


@pytest.mark.parametrize("mirror,ctype", [(_lib.NormArgs, "arn_norm_args"),
                                          (_lib.SumNormArgs, "arn_sum_norm_args")])
def test_norm_struct_layout_matches_header(mirror, ctype):
    """Field offsets of the ctypes mirror equal those of the C struct,
    measured by compiling a probe against include/arn.h with the host
    compiler (no GPU code)."""
    import tempfile
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"arn.h\"\nint main(void){\n"
    for name, _ in mirror._fields_:
        src += f'  printf("{name} %zu\\n", offsetof({ctype}, {name}));\n'
    src += f'  printf("size %zu\\n", sizeof({ctype}));\n  return 0;\n}}\n'
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "probe")
        subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = dict(zip(out[0::2], map(int, out[1::2])))
    for name, _ in mirror._fields_:
        assert got[name] == getattr(mirror, name).offset, name
    assert got["size"] == ctypes.sizeof(mirror)


def _sum_args(**kw):
    ptrs = (ctypes.c_void_p * 8)(*([Q] * 8))
    a = _lib.SumNormArgs(struct_size=ctypes.sizeof(_lib.SumNormArgs), dtype=0, out_format=0,
                         out=P, out_stride=64, scale=None,
                         parts=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), nparts=2,
                         parts_stride=64, residual=R, residual_stride=64, weight=None, eps=1e-6,
                         rows=4, hidden=64, stream=None)
    a._keep = ptrs
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("case", [
    dict(struct_size=8), dict(out_format=3), dict(nparts=0), dict(nparts=9),
    dict(parts=None), dict(out_format=1, scale=None), dict(parts_stride=10), dict(dtype=3),
])
def test_sum_descriptor_rejects(lib, case):
    a = _sum_args(**case)
    assert lib.arn_sum_add_rmsnorm(ctypes.byref(a)) == _lib.EINVAL
    assert lib.arn_sum_add_rmsnorm(None) == _lib.EINVAL


def test_sum_descriptor_residual_aliasing_a_part(lib):
    ptrs = (ctypes.c_void_p * 2)(Q, R)
    a = _sum_args(parts=ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)))
    assert lib.arn_sum_add_rmsnorm(ctypes.byref(a)) == _lib.EINVAL


def test_noalloc_gemm_limits_and_refusals(lib):
    """The no-allocation GEMM serves exactly the shapes whose workspace fits
    its 8 MiB device array (the limits the header states) and refuses the
    others, and invalid arguments, before any HIP call."""
    cap = _lib.NOALLOC_SCRATCH_BYTES
    assert cap == 8 << 20
    for m, nmax in ((64, 4032), (32, 8128), (16, 16256), (1, 16256)):
        assert lib.arn_fp8_gemm_workspace_bytes(m, nmax, 4096) <= cap
        assert lib.arn_fp8_gemm_workspace_bytes(m, nmax + 1, 4096) > cap
    f = lib.arn_fp8_gemm_preshuffled_noalloc
    P = 1 << 20
    args = lambda m, n, k=256, dt=0, lda=256, ldc=None: (  # noqa: E731
        P, ldc if ldc is not None else n, dt, P, lda, P, 1, P, P, 1, m, n, k, None)
    assert f(*args(64, 4033)) == _lib.EUNSUPPORTED
    assert f(*args(16, 16257)) == _lib.EUNSUPPORTED
    assert f(*args(4, 64, dt=2)) == _lib.EINVAL
    assert f(*args(4, 64, lda=128)) == _lib.EINVAL
    assert f(*args(-1, 64)) == _lib.EINVAL
    assert f(*args(0, 64)) == _lib.OK and f(*args(4, 0)) == _lib.OK
    a = list(args(4, 64))
    a[0] = None
    assert f(*a) == _lib.EINVAL
