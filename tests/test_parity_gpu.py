"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case feeds the same seeded inputs to both sides and applies the
comparison rules in tests/_helpers.py.  Outputs start as NaN canaries, row
padding starts as a NaN sentinel and one guard row follows the last row, so
a kernel that drops stores, reads padding into a row's sum, or writes past
the last row fails.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import (assert_codes_close, assert_scales_close, assert_y_close,
                            bits, codes, dev, static_scale, values16)

pytestmark = pytest.mark.gpu

CANARY16 = 0x7FC1  # a NaN in bf16 and in fp16
CANARY8 = 0x7F     # the e4m3 NaN code


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import residual_add_rmsnorm_amd as arn

    arn.set_tile(0, 0)
    yield
    arn.set_tile(0, 0)


def _arn():
    import residual_add_rmsnorm_amd as arn

    return arn


def run_case(orc, *, dtype, x, res, w, eps, hidden, fp8=None, s=None, out_stride=None,
             alias_out=False):
    """x, res: (rows, stride) uint16 host arrays (padding included);
    w: (hidden,) uint16 or None.  Returns nothing; asserts parity."""
    arn = _arn()
    rows, stride = x.shape
    out_stride = out_stride or stride
    fused = res is not None

    # device buffers with one guard row each
    def with_guard(a, fill):
        g = np.full((rows + 1, a.shape[1]), fill, np.uint16)
        g[:rows] = a
        return g

    xd = dev(with_guard(x, W.PAD_SENTINEL), dtype)
    rd = dev(with_guard(res, W.PAD_SENTINEL), dtype) if fused else None
    wd = dev(w, dtype) if w is not None else None
    xv = xd[:rows, :hidden]
    rv = rd[:rows, :hidden] if fused else None

    if fp8:
        od = torch.full((rows + 1, out_stride), CANARY8, dtype=torch.uint8, device="cuda")
        ov = od.view(torch.float8_e4m3fn)[:rows, :hidden]
        if fp8 == "static":
            sd = torch.tensor([s], dtype=torch.float32, device="cuda")
            kw = dict(scale=sd)
        else:
            sd = torch.full((rows + 1,), float("nan"), dtype=torch.float32, device="cuda")
            kw = dict(dynamic=True, scales_out=sd[:rows])
        if fused:
            arn.fused_add_rmsnorm_fp8(xv, rv, wd, eps, out=ov, **kw)
        else:
            arn.rmsnorm_fp8(xv, wd, eps, out=ov, **kw)
    else:
        if alias_out:
            od, ov = xd, xv
        else:
            od = dev(np.full((rows + 1, out_stride), CANARY16, np.uint16), dtype)
            ov = od[:rows, :hidden]
        if fused:
            arn.fused_add_rmsnorm(xv, rv, wd, eps, out=ov)
        else:
            arn.rmsnorm(xv, wd, eps, out=ov)
    torch.cuda.synchronize()

    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.add_rmsnorm(dtype, x, res, w, eps, hidden=hidden, fp8_mode=mode,
                          static_scale=s or 0.0)

    if fused:
        rb = bits(rd)
        assert np.array_equal(rb[:rows, :hidden], ref["r16"]), "stored residual not bit-exact"
        assert np.all(rb[:rows, hidden:] == W.PAD_SENTINEL), "residual padding written"
        assert np.all(rb[rows] == W.PAD_SENTINEL), "residual guard row written"
    xb = bits(xd)
    if not alias_out:
        assert np.array_equal(xb[:rows], x), "x modified"
    assert np.all(xb[rows] == W.PAD_SENTINEL), "x guard row written"

    if fp8:
        q = codes(od)
        assert_codes_close(q[:rows, :hidden], ref["q"])
        assert np.all(q[:rows, hidden:] == CANARY8), "output padding written"
        assert np.all(q[rows] == CANARY8), "output guard row written"
        if fp8 == "dynamic":
            sc = sd.cpu().numpy()
            assert_scales_close(sc[:rows], ref["scales"], dtype)
            assert np.isnan(sc[rows]), "scale guard written"
    else:
        ob = bits(od)
        assert_y_close(ob[:rows, :hidden], ref["y"], dtype)
        if not alias_out:
            assert np.all(ob[:rows, hidden:] == CANARY16), "output padding written"
            assert np.all(ob[rows] == CANARY16), "output guard row written"


def _random(dtype, rows, hidden, stride, seed, std=1.0):
    rng = np.random.default_rng(seed)
    a = np.full((rows, stride), W.PAD_SENTINEL, np.uint16)
    a[:, :hidden] = W.to_bits((rng.standard_normal((rows, hidden)) * std).astype(np.float32), dtype)
    return a


# ---------------------------------------------------------------------------
# The five workloads at oracle-friendly sizes (several tiles + a ragged tail)
# ---------------------------------------------------------------------------

def _workload_case(orc, name, rows, **over):
    w = W.WORKLOADS[name]
    d = W.make(w, rows=rows)
    fp8 = w.fp8
    s = static_scale() if fp8 == "static" else None
    run_case(orc, dtype=w.dtype, x=d["x"], res=d.get("residual"), w=d["weight"],
             eps=w.eps, hidden=w.hidden, fp8=fp8, s=s, **over)


def test_rmsnorm_bf16_64x4096(orc):
    _workload_case(orc, "rmsnorm_bf16_64x4096", 64)


@pytest.mark.parametrize("rows", [1, 77, 512])
def test_fused_bf16_x8192(orc, rows):
    _workload_case(orc, "fused_add_rmsnorm_bf16_4096x8192", rows)


@pytest.mark.parametrize("rows", [1, 8, 64, 256])
def test_fused_fp8_static_fp16_decode(orc, rows):
    _workload_case(orc, "fused_add_rmsnorm_fp8_static_fp16_decode_x16384", rows)


@pytest.mark.parametrize("rows", [3, 300])
def test_fused_fp8_dynamic_bf16_x7168(orc, rows):
    _workload_case(orc, "fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168", rows)


@pytest.mark.parametrize("name", ["fused_add_rmsnorm_bf16_65536x3840_stride4096",
                                  "fused_add_rmsnorm_bf16_65536x2880_stride4096"])
@pytest.mark.parametrize("rows", [5, 1029])
def test_fused_strided_rows(orc, name, rows):
    _workload_case(orc, name, rows)


# ---------------------------------------------------------------------------
# Shapes, layouts and degenerate cases
# ---------------------------------------------------------------------------

HIDDENS = [1, 2, 3, 7, 8, 16, 31, 64, 100, 511, 512, 513, 1000, 2880, 3840, 4095, 4096, 5120,
           8192, 12288, 16384, 32768, 65536]


@pytest.mark.parametrize("hidden", HIDDENS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_hidden_sweep_fused(orc, dtype, hidden):
    rows = 3 if hidden > 8192 else 37
    x = _random(dtype, rows, hidden, hidden, 1)
    r = _random(dtype, rows, hidden, hidden, 2)
    w = _random(dtype, 1, hidden, hidden, 3)[0] if hidden % 3 else None
    run_case(orc, dtype=dtype, x=x, res=r, w=w, eps=1e-5, hidden=hidden)


@pytest.mark.parametrize("hidden", [1, 24, 513, 4096, 7168, 16384])
@pytest.mark.parametrize("fp8", ["static", "dynamic"])
@pytest.mark.parametrize("fused", [False, True])
def test_hidden_sweep_fp8(orc, hidden, fp8, fused):
    dtype = "bf16" if hidden % 2 else "fp16"
    rows = 5
    x = _random(dtype, rows, hidden, hidden, 4)
    r = _random(dtype, rows, hidden, hidden, 5) if fused else None
    w = _random(dtype, 1, hidden, hidden, 6)[0]
    run_case(orc, dtype=dtype, x=x, res=r, w=w, eps=1e-6, hidden=hidden, fp8=fp8,
             s=0.01 if fp8 == "static" else None)


@pytest.mark.parametrize("hidden,tile", [(1024, "wpr1/nv2/rpb4"), (2048, "wpr2/nv2/rpb2"),
                                         (2880, "wpr4/nv2/rpb1"), (5120, "wpr4/nv3/rpb1"),
                                         (7168, "wpr4/nv4/rpb1"), (12288, "wpr16/nv2/rpb1")])
@pytest.mark.parametrize("fp8", [None, "dynamic", "static"])
def test_plain_many_rows_automatic_tiles(orc, hidden, tile, fp8):
    """The plain kinds with many rows (at least 4 per CU) take rows of at
    most four waves with up to four vectors per lane, fewer waves for
    narrow rows; wider rows fall back to the general rule.  1030 rows
    (several rows per block where the tile holds more than one, and a
    ragged last block), every row against the oracle."""
    arn = _arn()
    rows = 4 * torch.cuda.get_device_properties(0).multi_processor_count + 6
    dtype = "bf16"
    x = _random(dtype, rows, hidden, hidden, 40 + hidden % 97)
    w = _random(dtype, 1, hidden, hidden, 41)[0]
    run_case(orc, dtype=dtype, x=x, res=None, w=w, eps=1e-6, hidden=hidden, fp8=fp8,
             s=0.01 if fp8 == "static" else None)
    assert f"/vec8/{tile}/" in arn.last_plan(), arn.last_plan()


@pytest.mark.parametrize("hidden,fused,fp8", [(1030, False, "dynamic"), (1028, True, "dynamic"),
                                              (2050, False, None), (3076, True, None)])
def test_many_rows_narrow_accesses(orc, hidden, fused, fp8):
    """Many rows whose width allows only 4- or 2-element accesses (the
    compact rule looks among those tiles, else the general rule); every row
    against the oracle."""
    rows = 4 * torch.cuda.get_device_properties(0).multi_processor_count + 7
    x = _random("bf16", rows, hidden, hidden, 80)
    r = _random("bf16", rows, hidden, hidden, 81) if fused else None
    w = _random("bf16", 1, hidden, hidden, 82)[0]
    run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=1e-6, hidden=hidden, fp8=fp8)


@pytest.mark.parametrize("hidden,tile", [(1024, "wpr1/nv2/rpb4"), (2048, "wpr2/nv2/rpb2"),
                                         (2880, "wpr4/nv2/rpb1"), (4096, "wpr4/nv2/rpb1"),
                                         (7168, "wpr8/nv2/rpb1")])
def test_fused_dynamic_many_rows_automatic_tiles(orc, hidden, tile):
    """The fused dynamic-e4m3 kind with many rows takes the compact tile up
    to two vectors per lane (rows up to 4096 wide) and the general rule
    beyond; every row of 4 x CUs + 5 rows against the oracle."""
    arn = _arn()
    rows = 4 * torch.cuda.get_device_properties(0).multi_processor_count + 5
    x = _random("bf16", rows, hidden, hidden, 70 + hidden % 83)
    r = _random("bf16", rows, hidden, hidden, 71)
    w = _random("bf16", 1, hidden, hidden, 72)[0]
    run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=1e-6, hidden=hidden, fp8="dynamic")
    assert f"/vec8/{tile}/" in arn.last_plan(), arn.last_plan()


@pytest.mark.parametrize("hidden,per_cu,dtype,tile", [
    (5120, 1.0, "fp16", "wpr4/nv3/rpb1"), (7168, 1.25, "bf16", "wpr4/nv4/rpb1"),
    (8192, 1.0, "fp16", "wpr4/nv4/rpb1"), (4104, 0.75, "bf16", "wpr4/nv3/rpb1"),
    (7168, 1.5, "bf16", "wpr2/nv8/rpb2"), (8192, 2.0, "fp16", "wpr2/nv8/rpb2"),
    (5120, 1.75, "bf16", "wpr4/nv3/rpb1"), (8192, 0.5, "bf16", "wpr8/nv2/rpb1"),
    (8192, 0.5, "fp16", "wpr4/nv4/rpb1"), (7168, 0.25, "fp16", "wpr4/nv4/rpb1"),
    (7168, 0.0, "fp16", "wpr4/nv4/rpb1"), (7168, 0.25, "bf16", "wpr8/nv2/rpb1"),
    (8192, 2.5, "fp16", "wpr8/nv2/rpb1"), (4096, 1.0, "fp16", "wpr8/nv1/rpb1"),
    (7168, 1.504, "bf16", "wpr2/nv8/rpb2")])  # 385 rows on 256 CUs: a half-empty last block
@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
def test_fused_rows_near_cu_count_automatic_tiles(orc, hidden, per_cu, dtype, tile, fp8):
    """Fused rows 4097-8192 wide with at most two rows per CU take four-wave
    rows up to one and a quarter rows per CU (at half a row per CU or fewer
    for fp16 only), then two-wave rows of eight vectors when the row has
    more than 768 vectors (four waves below that); bf16 rows at half a row
    per CU, two and a half rows per CU, and 4096-wide rows keep the
    eight-wave rule.  Every row against the oracle, plan asserted."""
    arn = _arn()
    rows = max(1, int(per_cu * torch.cuda.get_device_properties(0).multi_processor_count))
    x = _random(dtype, rows, hidden, hidden, 90 + hidden % 89)
    r = _random(dtype, rows, hidden, hidden, 91)
    w = _random(dtype, 1, hidden, hidden, 92)[0]
    run_case(orc, dtype=dtype, x=x, res=r, w=w, eps=1e-6, hidden=hidden, fp8=fp8,
             s=0.01 if fp8 == "static" else None)
    assert f"/vec8/{tile}/" in arn.last_plan(), arn.last_plan()


@pytest.mark.parametrize("rows", [1, 2, 255, 256, 257, 1025, 4099])
def test_row_counts(orc, rows):
    x = _random("bf16", rows, 1024, 1024, 7)
    r = _random("bf16", rows, 1024, 1024, 8)
    run_case(orc, dtype="bf16", x=x, res=r, w=None, eps=1e-6, hidden=1024)


@pytest.mark.parametrize("hidden,stride", [(96, 100), (4096, 4104), (1000, 1001), (384, 385)])
def test_odd_strides_fall_back_to_narrow_accesses(orc, hidden, stride):
    x = _random("fp16", 9, hidden, stride, 9)
    r = _random("fp16", 9, hidden, stride, 10)
    w = _random("fp16", 1, hidden, hidden, 11)[0]
    run_case(orc, dtype="fp16", x=x, res=r, w=w, eps=1e-5, hidden=hidden,
             out_stride=stride + 3)
    plan = _arn().last_plan()
    assert "vec8" not in plan, plan


def test_misaligned_base_pointer(orc):
    arn = _arn()
    rows, hidden = 6, 512
    x = _random("bf16", rows, hidden, hidden, 12)
    r = _random("bf16", rows, hidden, hidden, 13)
    buf = torch.zeros(rows * hidden + 1, dtype=torch.bfloat16, device="cuda")
    xv = buf[1:].view(rows, hidden)  # 2-byte aligned only
    xv.copy_(dev(x, "bf16"))
    rd = dev(r, "bf16")
    out = arn.fused_add_rmsnorm(xv, rd, None, 1e-6)
    torch.cuda.synchronize()
    assert "vec1" in arn.last_plan()
    ref = orc.add_rmsnorm("bf16", x, r, None, 1e-6)
    assert np.array_equal(bits(rd), ref["r16"])
    assert_y_close(bits(out), ref["y"], "bf16")


def test_out_aliases_x(orc):
    x = _random("bf16", 33, 2048, 2048, 14)
    r = _random("bf16", 33, 2048, 2048, 15)
    w = _random("bf16", 1, 2048, 2048, 16)[0]
    run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=1e-6, hidden=2048,
             alias_out=True)


def test_plain_out_aliases_x(orc):
    x = _random("fp16", 7, 4096, 4096, 17)
    run_case(orc, dtype="fp16", x=x, res=None, w=None, eps=1e-6, hidden=4096,
             alias_out=True)


def test_fp16_subnormal_inputs(orc):
    rng = np.random.default_rng(18)
    rows, hidden = 8, 1024
    f = (rng.standard_normal((rows, hidden)) * 2.0**-18).astype(np.float32)  # mostly subnormal
    x = W.to_bits(f, "fp16")
    r = W.to_bits(-0.5 * f, "fp16")
    run_case(orc, dtype="fp16", x=x, res=r, w=None, eps=0.0, hidden=hidden)


# Rows at both ends of bf16's range, interleaved with ordinary ones so that
# blocks holding several rows mix them.  With a small eps the fp32 sum of
# squares of such rows underflows (every |r| below about 2^-75: squares
# under fp32's smallest values) or overflows (|r| of 2^60 and more over a
# 2048-wide row); the kernel recomputes it from r scaled by 2^+-76, so these
# rows meet the same tolerance as any other.
OUT_OF_RANGE_SCALES = [2.0**-131, 1.0, 2.0**-128, 2.0**-100, 1e-3, 1e-30, 2.0**-80,
                       2.0**-70, 2.0**60, 1.0, 2.0**100, 2.0**124, 2.0**-40, 3.0]


def _out_of_range_rows(hidden=2048, seed=19):
    rng = np.random.default_rng(seed)
    sc = np.array(OUT_OF_RANGE_SCALES, np.float64)
    f = rng.standard_normal((sc.size, hidden)) * sc[:, None]
    f = np.clip(f, -2.0**126, 2.0**126).astype(np.float32)
    x = W.to_bits(f, "bf16")
    r = W.to_bits(f * np.float32(0.25), "bf16")
    w = W.to_bits(rng.uniform(0.5, 1.5, hidden).astype(np.float32), "bf16")
    return x, r, w


@pytest.mark.parametrize("tile", [None, (1, 4), (2, 2), (8, 1), (16, 1)],
                         ids=["auto", "wpr1", "wpr2", "wpr8", "wpr16"])
@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
@pytest.mark.parametrize("eps", [0.0, 1e-38, 1e-6])
def test_bf16_rows_out_of_fp32_range(orc, eps, fp8, tile):
    """Subnormal, tiny and huge bf16 rows (their squares or sums of squares
    out of fp32's range) match the fp64 definition, with eps = 0, an eps far
    below them, or an ordinary eps; every output format; one-row-per-wave,
    two-rows-per-block and multi-wave tiles forced."""
    arn = _arn()
    x, r, w = _out_of_range_rows()
    hidden = x.shape[1]
    if tile:
        arn.set_tile(*tile)
    try:
        run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=eps, hidden=hidden, fp8=fp8,
                 s=2.0**-6 if fp8 == "static" else None)
        if tile:
            assert f"/wpr{tile[0]}/nv{tile[1]}/" in arn.last_plan()
    finally:
        arn.set_tile(0, 0)


@pytest.mark.parametrize("k", [2048, 700])
def test_bf16_rows_out_of_fp32_range_variance_size(orc, k):
    arn = _arn()
    x, r, w = _out_of_range_rows(seed=23)
    H = x.shape[1]
    xd, rd, wd = dev(x, "bf16"), dev(r, "bf16"), dev(w, "bf16")
    y = arn.norm(xd, wd, 0.0, residual=rd, variance_size=k)
    torch.cuda.synchronize()
    ref = orc.add_rmsnorm("bf16", x, r, w, 0.0, variance_size=k)
    assert np.array_equal(bits(rd), ref["r16"])
    assert_y_close(bits(y), ref["y"], "bf16")


# Dynamic e4m3 rows whose products r * w leave fp32's range although their
# sums of squares may not: tiny weights under ordinary activations, huge
# weights under large activations, both tiny (the scale then underflows to an
# fp32 subnormal or to zero), and a single product past 2^128.  Each family
# is one weight vector; the rows vary the activations' magnitude.  Values
# are drawn away from zero (|v| = scale * U(1, 2), random sign), so no y is
# exactly zero where the scale rounds to zero (0 / 0 there); the residual
# takes x's signs, so x + residual does not cancel.
WIDE_WEIGHTS = {
    "tiny_w": (2.0**-120, [1.0, 2.0**30, 2.0**-60, 2.0**-131, 2.0**10]),
    "denormal_w": (2.0**-130, [2.0**-131, 1.0, 2.0**40, 2.0**-100, 2.0**90]),
    "huge_w": (2.0**80, [2.0**50, 2.0**60, 1.0, 2.0**-131, 2.0**-100]),
    "mixed_w": (None, [1.0, 2.0**100, 2.0**-120, 2.0**40, 2.0**-131]),
}


def _wide_rows(family, hidden, seed):
    """(x, residual, w) bit patterns for one family of WIDE_WEIGHTS."""
    rng = np.random.default_rng(seed)
    wscale, xscales = WIDE_WEIGHTS[family]

    def mag(n, scale):
        return np.minimum(scale * rng.uniform(1.0, 2.0, n), 2.0**127)

    if wscale is None:  # one huge, one tiny and one subnormal column among ordinary ones
        wf = rng.uniform(0.5, 1.5, hidden)
        wf[[3, hidden // 2, hidden - 1]] = [2.0**100, 2.0**-125, 2.0**-132]
    else:
        wf = mag(hidden, wscale)
    sign = np.where(rng.random((len(xscales), hidden)) < 0.5, -1.0, 1.0)
    xf = sign * np.stack([mag(hidden, sc) for sc in xscales])
    rf = sign * np.stack([mag(hidden, sc) for sc in xscales])
    return tuple(W.to_bits(a.astype(np.float32), "bf16") for a in (xf, rf, wf))


@pytest.mark.parametrize("tile", [None, (1, 4), (2, 2), (8, 1), (16, 1)],
                         ids=["auto", "wpr1", "wpr2", "wpr8", "wpr16"])
@pytest.mark.parametrize("eps", [0.0, 1e-6])
@pytest.mark.parametrize("family", list(WIDE_WEIGHTS))
def test_bf16_dynamic_products_out_of_fp32_range(orc, family, eps, tile):
    """Codes and scales of rows whose products overflow fp32 or fall below
    2^-96 (down to products under 2^-256 whose scale rounds to zero) match
    the fp64 definition; with and without the residual, every tile shape
    (one-row-per-wave, two rows per block sharing a barrier, multi-wave)."""
    arn = _arn()
    hidden = 2048
    x, r, w = _wide_rows(family, hidden, seed=31)
    if tile:
        arn.set_tile(*tile)
    try:
        run_case(orc, dtype="bf16", x=x, res=None, w=w, eps=eps, hidden=hidden, fp8="dynamic")
        run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=eps, hidden=hidden, fp8="dynamic")
        if tile:
            assert f"/wpr{tile[0]}/nv{tile[1]}/" in arn.last_plan()
    finally:
        arn.set_tile(0, 0)


def test_zero_rows_eps0_give_nan(orc):
    x = np.zeros((4, 256), np.uint16)
    run_case(orc, dtype="bf16", x=x, res=None, w=None, eps=0.0, hidden=256)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("variance", [None, 500])
def test_nonfinite_inputs_propagate(orc, dtype, fused, variance):
    """Infinities and NaNs in the activations follow IEEE arithmetic through
    the definition: a NaN in the mean makes the whole row NaN; an infinity
    there makes the mean infinite, so every finite channel comes out as a
    signed zero and the infinite one as NaN (inf * 0); an infinity outside a
    smaller variance size passes through as an infinite output; +inf plus
    -inf in the residual add stores a NaN.  16-bit outputs (e4m3 codes of
    non-finite y are not specified).  NaN bit patterns are not compared,
    only where they are."""
    arn = _arn()
    hidden, rows = 1000, 7
    inf, nan = (0x7F80, 0x7FC0) if dtype == "bf16" else (0x7C00, 0x7E00)
    x = _random(dtype, rows, hidden, hidden, 70)
    r = _random(dtype, rows, hidden, hidden, 71)
    x[0, 3] = inf
    x[1, 10] = nan
    (r if fused else x)[2, 20] = inf | 0x8000
    x[3, 30] = inf
    r[3, 30] = inf | 0x8000  # with the residual: +inf + -inf = NaN
    x[5, hidden - 1] = inf  # the ragged tail, past a variance size of 500
    x[6, 600] = nan | 0x8000
    xd, wd = dev(x, dtype), dev(_random(dtype, 1, hidden, hidden, 72)[0], dtype)
    w = bits(wd)
    rd = dev(r, dtype) if fused else None
    out = arn.norm(xd, wd, 0.0, residual=rd, variance_size=variance)
    torch.cuda.synchronize()
    ref = orc.add_rmsnorm(dtype, x, r if fused else None, w, 0.0, variance_size=variance)
    if fused:
        got = values16(bits(rd), dtype)
        want = values16(ref["r16"], dtype)
        assert np.array_equal(np.isnan(got), np.isnan(want)), "residual NaN positions differ"
        keep = ~np.isnan(want)
        assert np.array_equal(bits(rd)[keep], ref["r16"][keep]), "stored residual not bit-exact"
    assert np.isnan(ref["y"][1]).all()
    if variance:
        assert np.isinf(ref["y"][5, hidden - 1]) and np.isfinite(ref["y"][5, :-1]).all()
    assert_y_close(bits(out), ref["y"], dtype)


def test_zero_rows_dynamic_fp8(orc):
    x = _random("bf16", 6, 768, 768, 20)
    r = _random("bf16", 6, 768, 768, 21)
    x[2] = 0
    r[2] = 0
    x[4] = 0x8000  # -0 + -0 = -0
    r[4] = 0x8000
    run_case(orc, dtype="bf16", x=x, res=r, w=None, eps=1e-6, hidden=768,
             fp8="dynamic")


def test_fp8_static_saturates(orc):
    x = _random("fp16", 4, 2048, 2048, 22, std=4.0)
    run_case(orc, dtype="fp16", x=x, res=None, w=None, eps=1e-6, hidden=2048,
             fp8="static", s=1.0 / 256)


def _magnitude_rows(dtype, hidden, seed):
    """Rows of one magnitude each: ordinary, the dtype's smallest normal and
    subnormal values, its largest, and a row with exact zeros."""
    rng = np.random.default_rng(seed)
    big = 2.0**126 if dtype == "bf16" else 30000.0  # x + residual stays finite
    tiny = 2.0**-126 if dtype == "bf16" else 2.0**-14
    sub = 2.0**-131 if dtype == "bf16" else 2.0**-20
    rows = []
    for sc in (1.0, tiny, sub, big):
        rows.append(np.where(rng.random(hidden) < 0.5, -1.0, 1.0) * sc * rng.uniform(0.5, 1.0, hidden))
    z = rng.standard_normal(hidden)
    z[::3] = 0.0
    rows.append(z)
    return W.to_bits(np.stack(rows).astype(np.float32), dtype)


@pytest.mark.parametrize("s", [2.0**-126, 1e-30, 1e-6, 1.0, 1e30, 3.4e38])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp8_static_scale_range(orc, dtype, s):
    """Static e4m3 over the range of normal fp32 scales, on rows of every
    magnitude the dtype holds (zeros included): saturation at one end, codes
    rounding to zero at the other, both signs."""
    hidden = 1024
    x = _magnitude_rows(dtype, hidden, 70)
    r = _magnitude_rows(dtype, hidden, 71)
    w = W.to_bits(np.random.default_rng(72).uniform(0.25, 2.0, hidden).astype(np.float32), dtype)
    run_case(orc, dtype=dtype, x=x, res=None, w=w, eps=1e-6, hidden=hidden, fp8="static", s=s)
    run_case(orc, dtype=dtype, x=x, res=r, w=w, eps=0.0, hidden=hidden, fp8="static", s=s)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp8_dynamic_every_magnitude(orc, dtype):
    hidden = 1024
    x = _magnitude_rows(dtype, hidden, 73)
    r = _magnitude_rows(dtype, hidden, 74)
    w = W.to_bits(np.random.default_rng(75).uniform(0.25, 2.0, hidden).astype(np.float32), dtype)
    run_case(orc, dtype=dtype, x=x, res=None, w=w, eps=1e-6, hidden=hidden, fp8="dynamic")
    run_case(orc, dtype=dtype, x=x, res=r, w=w, eps=0.0, hidden=hidden, fp8="dynamic")


def test_zero_rows_launch_nothing():
    arn = _arn()
    x = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    r = torch.empty(0, 128, dtype=torch.bfloat16, device="cuda")
    out = arn.fused_add_rmsnorm(x, r, None, 1e-6)
    assert out.shape == (0, 128)


def test_3d_input_flattens(orc):
    arn = _arn()
    x = _random("bf16", 24, 640, 640, 23)
    r = _random("bf16", 24, 640, 640, 24)
    xd = dev(x, "bf16").view(4, 6, 640)
    rd = dev(r, "bf16").view(4, 6, 640)
    out = arn.fused_add_rmsnorm(xd, rd, None, 1e-6)
    torch.cuda.synchronize()
    ref = orc.add_rmsnorm("bf16", x, r, None, 1e-6)
    assert np.array_equal(bits(rd).reshape(24, 640), ref["r16"])
    assert_y_close(bits(out).reshape(24, 640), ref["y"], "bf16")


def test_deterministic():
    arn = _arn()
    x = dev(_random("bf16", 300, 7168, 7168, 25), "bf16")
    r0 = dev(_random("bf16", 300, 7168, 7168, 26), "bf16")
    outs = []
    for _ in range(2):
        r = r0.clone()
        q, s = arn.fused_add_rmsnorm_fp8(x, r, None, 1e-6, dynamic=True)
        y = arn.fused_add_rmsnorm(x, r0.clone(), None, 1e-6)
        torch.cuda.synchronize()
        outs.append((codes(q), s.cpu().numpy(), bits(y), bits(r)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


# ---------------------------------------------------------------------------
# Every compiled 128-bit kernel shape, forced
# ---------------------------------------------------------------------------

TILES_VEC8 = [(1, 2), (1, 4), (1, 8), (1, 16), (2, 2), (2, 4), (2, 8), (4, 1), (4, 2), (4, 3),
              (4, 4), (4, 8), (8, 1), (8, 2), (8, 4), (8, 8), (16, 1), (16, 2), (16, 4), (16, 8)]


@pytest.mark.parametrize("wpr,nv", TILES_VEC8)
@pytest.mark.parametrize("kind", ["fused", "dynamic"])
def test_forced_tiles(orc, wpr, nv, kind):
    arn = _arn()
    cover = 64 * wpr * nv * 8
    hidden = cover - 24  # every per-lane slot used, ragged last vectors
    x = _random("bf16", 11, hidden, hidden, 27)
    r = _random("bf16", 11, hidden, hidden, 28)
    w = _random("bf16", 1, hidden, hidden, 29)[0]
    arn.set_tile(wpr, nv)
    try:
        run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=1e-6, hidden=hidden,
                 fp8="dynamic" if kind == "dynamic" else None)
        assert f"wpr{wpr}/nv{nv}/" in arn.last_plan()
    finally:
        arn.set_tile(0, 0)


def test_forced_tile_too_small_is_unsupported():
    arn = _arn()
    x = torch.zeros(2, 4096, dtype=torch.bfloat16, device="cuda")
    arn.set_tile(1, 2)
    try:
        with pytest.raises(arn.ArnError) as e:
            arn.rmsnorm(x, None, 1e-6)
        assert e.value.status == 2
    finally:
        arn.set_tile(0, 0)


# ---------------------------------------------------------------------------
# The e4m3 conversion, exhaustively, through the ABI
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("log2s", [0, -4, 3])
def test_e4m3_conversion_every_16bit_weight(orc, dtype, log2s):
    """x = 1 in every channel and eps = 0 make the normaliser exactly 1, so
    y = w and the codes are e4m3(w / s) for every one of the 65536 16-bit
    weight patterns at once (hidden = 65536).  s is a power of two, so w / s
    is exact and the GPU's rounding and saturation must match the oracle's
    encoder code for code (NaN weights aside)."""
    arn = _arn()
    hidden = 65536
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    x = np.full((1, hidden), one, np.uint16)
    w = np.arange(hidden, dtype=np.uint32).astype(np.uint16)
    xd, wd = dev(x, dtype), dev(w, dtype)
    y = arn.rmsnorm(xd, wd, 0.0)
    s = 2.0**log2s
    q, _ = arn.rmsnorm_fp8(xd, wd, 0.0, scale=torch.tensor([s], device="cuda"))
    torch.cuda.synchronize()
    ref = orc.add_rmsnorm(dtype, x, None, w, 0.0, fp8_mode=O.FP8_STATIC, static_scale=s)
    finite = np.isfinite(ref["y"][0])
    # normaliser exactly 1: y reproduces the weight bit for bit
    assert np.array_equal(bits(y)[0][finite], w[finite])
    qg = codes(q)[0]
    mism = np.flatnonzero((qg != ref["q"][0]) & finite)
    assert mism.size == 0, (f"{mism.size} codes differ; first w={w[mism[0]]:#06x} "
                            f"gpu={qg[mism[0]]:#04x} ref={ref['q'][0][mism[0]]:#04x}")
    # +-Inf weights saturate
    inf = np.isinf(ref["y"][0])
    assert np.all((qg[inf] & 0x7F) == 0x7E)


def _fp32_with_reciprocal(q32):
    """An fp32 s whose correctly rounded fp32 reciprocal 1.0f / s is q32."""
    s = np.float32(1.0 / np.float64(q32))
    for _ in range(8):
        r = np.float32(1.0) / s
        if r == q32:
            return s
        s = np.nextafter(s, np.float32(np.inf) if r > q32 else np.float32(0))
    raise AssertionError(f"no fp32 scale with reciprocal {q32!r}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_e4m3_convert_near_ties_at_fp32_resolution(orc, dtype):
    """The packed convert rounds fp32 values, not only 16-bit ones.  x = 1,
    eps = 0 and a power-of-two width make the normaliser exactly 1, so the
    static kernel converts fp32(w * q) with q = 1.0f / s.  With q = 1 + j 2^-23
    (j = -3..3) and w every e4m3 rounding tie, every e4m3 value and the
    saturation edge, both signs, the converted values sit on a tie or a few
    fp32 ulps to either side of it.  Each code must be the nearest e4m3
    (ties to even, saturating at 448) of the fp32 value the kernel forms,
    which the host computes with numpy's float32 product."""
    arn = _arn()
    pos = sorted({orc.e4m3_decode(c) for c in range(0x7F)})         # 0 .. 448
    mids = [(lo + hi) / 2 for lo, hi in zip(pos[:-1], pos[1:])] + [464.0]
    vals = np.array(pos[1:] + mids, np.float64)
    vals = np.concatenate([vals, -vals])
    hidden = 1024
    assert vals.size <= hidden
    w16 = np.zeros(hidden, np.uint16)
    if dtype == "fp16":
        w16[:vals.size] = vals.astype(np.float16).view(np.uint16)
        wv = w16.view(np.float16).astype(np.float32)
    else:
        w16[:vals.size] = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        wv = torch.from_numpy(w16.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(wv[:vals.size].astype(np.float64), vals)  # every tie is a 16-bit value
    one = 0x3F80 if dtype == "bf16" else 0x3C00
    xd = dev(np.full((1, hidden), one, np.uint16), dtype)
    wd = dev(w16, dtype)
    enc = np.vectorize(lambda v: orc.e4m3_encode(float(v)), otypes=[np.uint8])
    for j in range(-3, 4):
        q32 = np.float32(1.0 + j * 2.0**-23)
        s = _fp32_with_reciprocal(q32)
        y32 = wv * q32                                              # fp32 products, RNE
        want = enc(y32.astype(np.float64))
        q, _ = arn.rmsnorm_fp8(xd, wd, 0.0, scale=torch.tensor([float(s)], device="cuda"))
        got = codes(q)[0]
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"j={j}: {bad.size} codes differ; first y={float(y32[bad[0]])!r} "
                               f"gpu={got[bad[0]]:#04x} want={want[bad[0]]:#04x}")


def test_e4m3_dynamic_every_finite_bf16_weight(orc):
    arn = _arn()
    w = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(w.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    w = w[np.isfinite(vals) & (np.abs(vals) < 1e30)]
    w = w[: (w.size // 8) * 8]
    hidden = w.size
    x = np.full((1, hidden), 0x3F80, np.uint16)
    run_case(orc, dtype="bf16", x=x, res=None, w=w, eps=0.0, hidden=hidden,
             fp8="dynamic")


# ---------------------------------------------------------------------------
# arn_norm: the descriptor entry point and the variance-size override
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hidden,k", [(4096, 4096), (4096, 1000), (4096, 1), (3840, 2048),
                                      (100, 37), (16384, 12288)])
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("fp8", [None, "dynamic"])
def test_norm_variance_size(orc, hidden, k, fused, fp8):
    arn = _arn()
    dtype = "bf16"
    rows = 9
    x = _random(dtype, rows, hidden, hidden, 60)
    r = _random(dtype, rows, hidden, hidden, 61)
    w = _random(dtype, 1, hidden, hidden, 62)[0]
    xd, rd, wd = dev(x, dtype), dev(r, dtype), dev(w, dtype)
    out = arn.norm(xd, wd, 1e-6, residual=rd if fused else None, variance_size=k, fp8=fp8)
    torch.cuda.synchronize()
    mode = O.FP8_DYNAMIC if fp8 else O.FP8_NONE
    ref = orc.add_rmsnorm(dtype, x, r if fused else None, w, 1e-6, fp8_mode=mode,
                          variance_size=k)
    if fused:
        assert np.array_equal(bits(rd), ref["r16"])
    if fp8:
        q, sc = out
        assert_codes_close(codes(q), ref["q"])
        assert_scales_close(sc.cpu().numpy(), ref["scales"], dtype)
    else:
        assert_y_close(bits(out), ref["y"], dtype)


# (mean-square channels, other channels, static scale), as powers of two.
# The row factor 1/rms is 2^60 (a normal number after the rescaled sum),
# 2^130 (past fp32's largest value) and about 2^-127.5 (subnormal).
FAR_APART = {
    "tiny_mean": (-60, 60, 115),
    "subnormal_mean": (-130, -25, 100),
    "huge_mean": (127, 100, -30),
}


@pytest.mark.parametrize("k", [1, 3])
@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
@pytest.mark.parametrize("regime", sorted(FAR_APART))
def test_norm_variance_size_far_apart_channels(orc, regime, k, fp8):
    """A variance size k below the row, with the k channels the mean runs
    over and the other channels far apart in magnitude, so the sum of
    squares needs the rescaled recomputation while r times the row factor
    stays in range for the other channels: neither the scaled sum nor y may
    pass through an out-of-range intermediate (2^60 * 2^76 overflows).
    With tiny mean-square channels under 2^100 channels, y passes 448 times
    fp32's largest value, so the dynamic scale is +inf and every code is
    E(y / inf) = +-0, as in the definition."""
    arn = _arn()
    rng = np.random.default_rng(66)
    lv, lo, ls = FAR_APART[regime]
    if regime == "tiny_mean" and fp8 == "dynamic":
        lo = 100
    hidden, rows = 512, 3
    sign = np.where(rng.random((rows, hidden)) < 0.5, -1.0, 1.0)
    f = sign * 2.0**lo * rng.uniform(1, 2, (rows, hidden))
    f[:, :k] = sign[:, :k] * 2.0**lv * rng.uniform(1, 1.9, (rows, k))
    wf = rng.uniform(0.5, 1.5, hidden)
    x = W.to_bits(f.astype(np.float32), "bf16")
    w = W.to_bits(wf.astype(np.float32), "bf16")
    xd, wd = dev(x, "bf16"), dev(w, "bf16")
    s = 2.0**ls
    kw = dict(fp8="dynamic") if fp8 == "dynamic" else (
        dict(fp8="static", scale=torch.tensor([s], device="cuda")) if fp8 else {})
    out = arn.norm(xd, wd, 0.0, variance_size=k, **kw)
    torch.cuda.synchronize()
    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.add_rmsnorm("bf16", x, None, w, 0.0, fp8_mode=mode, static_scale=s,
                          variance_size=k)
    if fp8 == "dynamic":
        q, sc = out
        if regime == "tiny_mean":
            assert np.all(np.isinf(ref["scales"]))
        assert_scales_close(sc.cpu().numpy(), ref["scales"], "bf16")
        assert_codes_close(codes(q), ref["q"])
    elif fp8 == "static":
        assert_codes_close(codes(out[0]), ref["q"])
    else:
        assert np.all(np.abs(ref["y"]) < 2.0**127)
        assert_y_close(bits(out), ref["y"], "bf16")


@pytest.mark.parametrize("hidden,k,fused,fp8,tile", [
    (5120, 1000, False, None, "wpr4/nv3/rpb1"), (2048, 2047, False, "dynamic", "wpr2/nv2/rpb2"),
    (2880, 2000, True, "dynamic", "wpr4/nv2/rpb1"), (7168, 4096, True, None, "wpr8/nv2/rpb1")])
def test_norm_variance_size_many_rows(orc, hidden, k, fused, fp8, tile):
    """The variance-size override on the tiles many rows get (compact and
    eight-wave), every row of 4 x CUs + 1 rows against the oracle."""
    arn = _arn()
    dtype = "bf16"
    rows = 4 * torch.cuda.get_device_properties(0).multi_processor_count + 1
    x = _random(dtype, rows, hidden, hidden, 63)
    r = _random(dtype, rows, hidden, hidden, 64)
    w = _random(dtype, 1, hidden, hidden, 65)[0]
    xd, rd, wd = dev(x, dtype), dev(r, dtype), dev(w, dtype)
    out = arn.norm(xd, wd, 1e-6, residual=rd if fused else None, variance_size=k, fp8=fp8)
    torch.cuda.synchronize()
    assert f"/vec8/{tile}/" in arn.last_plan(), arn.last_plan()
    mode = O.FP8_DYNAMIC if fp8 else O.FP8_NONE
    ref = orc.add_rmsnorm(dtype, x, r if fused else None, w, 1e-6, fp8_mode=mode,
                          variance_size=k)
    if fused:
        assert np.array_equal(bits(rd), ref["r16"])
    if fp8:
        q, sc = out
        assert_codes_close(codes(q), ref["q"])
        assert_scales_close(sc.cpu().numpy(), ref["scales"], dtype)
    else:
        assert_y_close(bits(out), ref["y"], dtype)


def test_norm_descriptor_matches_entry_points(orc):
    arn = _arn()
    x = _random("fp16", 33, 2048, 2048, 63)
    r = _random("fp16", 33, 2048, 2048, 64)
    xd, r1, r2 = dev(x, "fp16"), dev(r, "fp16"), dev(r, "fp16")
    a = arn.fused_add_rmsnorm(xd, r1, None, 1e-5)
    b = arn.norm(xd, None, 1e-5, residual=r2)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a), bits(b)) and np.array_equal(bits(r1), bits(r2))


# ---------------------------------------------------------------------------
# The largest rows each access width serves, and the first size beyond
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("hidden,served", [
    (65536, True), (65544, False),   # 128-bit accesses: 16 waves x 8 vectors x 8 elements
    (65532, True), (65540, False),   # hidden % 8 == 4: 64-bit accesses, 16 x 16 x 4
    (32766, True), (32770, False),   # hidden % 4 == 2: 32-bit accesses, 16 x 16 x 2
    (16383, True), (16385, False),   # odd hidden: 16-bit accesses, 16 x 16 x 1
])
def test_largest_rows(orc, hidden, served):
    arn = _arn()
    rows = 2
    x = _random("bf16", rows, hidden, hidden, 11)
    r = _random("bf16", rows, hidden, hidden, 12)
    w = _random("bf16", 1, hidden, hidden, 13)[0]
    if served:
        run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=1e-6, hidden=hidden)
        run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=1e-6, hidden=hidden, fp8="dynamic")
        return
    xd, rd, wd = dev(x, "bf16"), dev(r, "bf16"), dev(w, "bf16")
    out = torch.full((rows, hidden), 7.0, dtype=torch.bfloat16, device="cuda")
    for call in (lambda: arn.fused_add_rmsnorm(xd, rd, wd, 1e-6, out=out),
                 lambda: arn.rmsnorm(xd, wd, 1e-6, out=out),
                 lambda: arn.fused_add_rmsnorm_fp8(xd, rd, wd, 1e-6, dynamic=True),
                 lambda: arn.silu_and_mul(torch.cat([xd, rd], dim=1))):
        with pytest.raises(arn.ArnError) as e:
            call()
        assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.equal(bits_t(rd), bits_t(dev(r, "bf16"))), "residual changed by a refused call"
    assert bool((out == 7.0).all()), "output written by a refused call"


def bits_t(t):
    return t.view(torch.int16)
