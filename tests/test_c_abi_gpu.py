"""The C boundary by itself: a plain C program (tests/c_abi/arn_client.c,
host code built with gcc against include/arn.h, no Python or torch in its
process) allocates device memory with hipMalloc, calls the library's entry
points (the norm in every output mode, the all-reduce form, SwiGLU, the
e4m3 GEMM in both weight layouts and with a split-K workspace) on a HIP
stream it created, and writes the results to a file; they must match the
oracle by the same rules as the Python-driven tests."""
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import (assert_codes_close, assert_scales_close, assert_y_close, gemm_ref, gemm_tol,
                            static_scale, values16)
from tests.c_abi import build as client_build

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def client():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return client_build.ensure()


def _run(client, args, tmp_path):
    print("arn_client", " ".join(str(a) for a in args), flush=True)
    res = subprocess.run([client, *[str(a) for a in args]], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr


def _inputs(rng, rows, hidden, stride, dtype, res_std=1.0):
    x = np.full((rows, stride), W.PAD_SENTINEL, np.uint16)
    r = np.full((rows, stride), W.PAD_SENTINEL, np.uint16)
    x[:, :hidden] = W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), dtype)
    r[:, :hidden] = W.to_bits((rng.standard_normal((rows, hidden)) * res_std).astype(np.float32),
                              dtype)
    w = W.to_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), dtype)
    return x, r, w


NORM_CASES = [
    # form, fp8, dtype, rows, hidden, stride, eps, variance_size
    ("fused", "none", "bf16", 37, 8192, 8200, 1e-5, 0),
    ("fused", "dynamic", "bf16", 33, 7168, 7168, 1e-6, 0),
    ("fused", "static", "fp16", 8, 16384, 16384, 1e-5, 0),
    ("plain", "none", "bf16", 64, 4096, 4096, 1e-6, 0),
    ("plain", "dynamic", "fp16", 5, 3840, 4096, 1e-6, 0),
    ("fused", "none", "bf16", 9, 4096, 4096, 1e-6, 2048),      # arn_norm, variance size
    ("plain", "static", "bf16", 6, 2880, 2880, 1e-6, 1000),    # arn_norm, variance size
]


@pytest.mark.parametrize("form,fp8,dtype,rows,hidden,stride,eps,var", NORM_CASES)
def test_norm_from_c(client, orc, tmp_path, form, fp8, dtype, rows, hidden, stride, eps, var):
    rng = np.random.default_rng(rows * 131 + hidden)
    fused = form == "fused"
    x, r, w = _inputs(rng, rows, hidden, stride, dtype, res_std=2.0 if dtype == "fp16" else 1.0)
    s = static_scale() if fp8 == "static" and dtype == "fp16" else (0.01 if fp8 == "static" else 0.0)
    s = float(np.float32(s))
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        f.write(x.tobytes())
        if fused:
            f.write(r.tobytes())
        f.write(w.tobytes())
    _run(client, ["norm", form, fp8, dtype, rows, hidden, stride, repr(eps), repr(s), var,
                  fin, fout], tmp_path)

    raw = open(fout, "rb").read()
    pos = 0
    n16 = rows * stride * 2
    if fused:
        r_after = np.frombuffer(raw[pos:pos + n16], np.uint16).reshape(rows, stride)
        pos += n16
    if fp8 == "none":
        out = np.frombuffer(raw[pos:pos + n16], np.uint16).reshape(rows, stride)
        pos += n16
    else:
        out = np.frombuffer(raw[pos:pos + rows * stride], np.uint8).reshape(rows, stride)
        pos += rows * stride
    scales = np.frombuffer(raw[pos:pos + 4 * rows], np.float32) if fp8 == "dynamic" else None

    mode = {"none": O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.add_rmsnorm(dtype, x, r if fused else None, w, eps, hidden=hidden, fp8_mode=mode,
                          static_scale=s, variance_size=var or None)
    if fused:
        assert np.array_equal(r_after[:, :hidden], ref["r16"]), "stored residual"
        assert np.all(r_after[:, hidden:] == W.PAD_SENTINEL), "residual padding touched"
    if fp8 == "none":
        assert_y_close(out[:, :hidden], ref["y"], dtype)
        assert np.all(out[:, hidden:] == 0), "output padding touched"
    else:
        assert_codes_close(out[:, :hidden], ref["q"])
        assert np.all(out[:, hidden:] == 0), "output padding touched"
    if scales is not None:
        assert_scales_close(scales, ref["scales"], dtype)


@pytest.mark.parametrize("layout", ["rowmajor", "preshuffled", "preshuffled_ws",
                                    "preshuffled_noalloc"])
def test_gemm_from_c(client, orc, tmp_path, layout):
    rng = np.random.default_rng(17)
    m, n, k = 9, 300, 1040   # few columns, M >= 8: with a workspace, K is split
    f = lambda rows, std: torch.from_numpy((rng.standard_normal((rows, k)) * std)
                                           .astype(np.float32)).clamp(-448, 448) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    a, b = f(m, 24.0), f(n, 6.0)
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as fh:
        for arr in (a, b, sa, sb):
            fh.write(np.ascontiguousarray(arr).tobytes())
    _run(client, ["gemm", layout, m, n, k, fin, fout], tmp_path)
    c = np.frombuffer(open(fout, "rb").read(), np.uint16).reshape(m, n)
    ref = gemm_ref(orc, a, sa, b, sb)
    got = values16(c, "bf16")
    tol = gemm_tol(ref, k)
    assert np.all(np.abs(got - ref["c"]) <= tol)


@pytest.mark.parametrize("fp8,dtype,nparts,rows,hidden,stride",
                         [("none", "bf16", 8, 6, 8192, 8192), ("dynamic", "bf16", 2, 9, 7168, 7176),
                          ("none", "fp16", 3, 5, 4096, 4104), ("dynamic", "fp16", 8, 4, 2880, 2880)])
def test_sum_from_c(client, orc, tmp_path, fp8, dtype, nparts, rows, hidden, stride):
    """arn_sum_add_rmsnorm from C: nparts partial rows (each in its own
    buffer) summed in rank order, added to the residual, normalised."""
    rng = np.random.default_rng(nparts * 1000 + hidden)
    std = nparts ** -0.5
    parts = []
    for _ in range(nparts):
        p = np.full((rows, stride), W.PAD_SENTINEL, np.uint16)
        p[:, :hidden] = W.to_bits((rng.standard_normal((rows, hidden)) * std).astype(np.float32),
                                  dtype)
        parts.append(p)
    _, r, w = _inputs(rng, rows, hidden, stride, dtype)
    eps = 1e-6
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(fin, "wb") as f:
        for p in parts:
            f.write(p.tobytes())
        f.write(r.tobytes())
        f.write(w.tobytes())
    _run(client, ["sum", fp8, dtype, nparts, rows, hidden, stride, repr(eps), fin, fout],
         tmp_path)
    raw = open(fout, "rb").read()
    n16 = rows * stride * 2
    r_after = np.frombuffer(raw[:n16], np.uint16).reshape(rows, stride)
    mode = O.FP8_DYNAMIC if fp8 == "dynamic" else O.FP8_NONE
    ref = orc.sum_add_rmsnorm(dtype, parts, r, w, eps, hidden=hidden, fp8_mode=mode)
    assert np.array_equal(r_after[:, :hidden], ref["r16"]), "stored residual"
    assert np.all(r_after[:, hidden:] == W.PAD_SENTINEL), "residual padding touched"
    if fp8 == "none":
        out = np.frombuffer(raw[n16:2 * n16], np.uint16).reshape(rows, stride)
        assert_y_close(out[:, :hidden], ref["y"], dtype)
    else:
        out = np.frombuffer(raw[n16:n16 + rows * stride], np.uint8).reshape(rows, stride)
        assert_codes_close(out[:, :hidden], ref["q"])
        scales = np.frombuffer(raw[n16 + rows * stride:], np.float32)
        assert_scales_close(scales, ref["scales"], dtype)
    assert np.all(out[:, hidden:] == 0), "output padding touched"


@pytest.mark.parametrize("fp8,dtype,rows,d", [("none", "bf16", 7, 6656), ("dynamic", "bf16", 5, 6656),
                                              ("dynamic", "fp16", 3, 2048)])
def test_glu_from_c(client, orc, tmp_path, fp8, dtype, rows, d):
    """arn_silu_and_mul(_fp8) from C on one [rows, 2d] gate/up tensor."""
    rng = np.random.default_rng(rows * 7 + d)
    gu = W.to_bits((rng.standard_normal((rows, 2 * d)) * 2).astype(np.float32), dtype)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(gu.tobytes())
    _run(client, ["glu", fp8, dtype, rows, d, fin, fout], tmp_path)
    raw = open(fout, "rb").read()
    mode = O.FP8_DYNAMIC if fp8 == "dynamic" else O.FP8_NONE
    ref = orc.silu_and_mul(dtype, gu, d=d, fp8_mode=mode)
    if fp8 == "none":
        out = np.frombuffer(raw, np.uint16).reshape(rows, d)
        assert_y_close(out, ref["y"], dtype)
    else:
        out = np.frombuffer(raw[:rows * d], np.uint8).reshape(rows, d)
        assert_codes_close(out, ref["q"])
        assert_scales_close(np.frombuffer(raw[rows * d:], np.float32), ref["scales"], dtype)


def test_client_reports_status(client, tmp_path):
    """An argument the library refuses comes back through arn_status_str."""
    fin = tmp_path / "in.bin"
    rows, hidden = 2, 100
    with open(fin, "wb") as f:
        f.write(np.zeros(rows * hidden * 2 + hidden, np.uint16).tobytes())
    # stride < hidden is invalid: the library returns ARN_EINVAL before any launch
    res = subprocess.run([client, "norm", "fused", "none", "bf16", str(rows), str(hidden),
                          str(hidden // 2), "1e-6", "0", "0", str(fin), str(tmp_path / "o.bin")],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 1
    assert "invalid argument" in res.stderr
