"""Parity of the SwiGLU (+ e4m3) HIP path with the oracle, through the C ABI.

out = silu(gate) * up with gate | up the two halves of a [rows, 2d] row
(the fused gate/up projection layout), or two separate tensors.  Outputs
start as NaN canaries and a guard row follows the last row.
"""

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import (assert_codes_close, assert_scales_close, assert_y_close, bits, codes,
                            dev, device_normal, static_scale)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import residual_add_rmsnorm_amd as arn

    arn.set_tile(0, 0)
    yield
    arn.set_tile(0, 0)


def _x(dtype, rows, d, stride=None, seed=50, std=2.0):
    stride = stride or 2 * d
    rng = np.random.default_rng(seed)
    a = np.full((rows, stride), W.PAD_SENTINEL, np.uint16)
    a[:, :2 * d] = W.to_bits((rng.standard_normal((rows, 2 * d)) * std).astype(np.float32), dtype)
    return a


def run_glu(orc, dtype, x, d, fp8=None, s=None):
    import residual_add_rmsnorm_amd as arn

    rows, stride = x.shape
    g = np.full((rows + 1, stride), W.PAD_SENTINEL, np.uint16)
    g[:rows] = x
    xd = dev(g, dtype)
    xv = xd[:rows, :2 * d]
    if fp8:
        od = torch.full((rows + 1, d), 0x7F, dtype=torch.uint8, device="cuda")
        ov = od.view(torch.float8_e4m3fn)[:rows]
        if fp8 == "static":
            sd = torch.tensor([s], dtype=torch.float32, device="cuda")
            arn.silu_and_mul_fp8(xv, scale=sd, out=ov)
        else:
            sd = torch.full((rows + 1,), float("nan"), dtype=torch.float32, device="cuda")
            arn.silu_and_mul_fp8(xv, dynamic=True, out=ov, scales_out=sd[:rows])
    else:
        od = dev(np.full((rows + 1, d), 0x7FC1, np.uint16), dtype)
        ov = od[:rows]
        arn.silu_and_mul(xv, out=ov)
    torch.cuda.synchronize()
    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.silu_and_mul(dtype, x, d=d, fp8_mode=mode, static_scale=s or 0.0)
    assert np.array_equal(bits(xd)[:rows], x), "input modified"
    if fp8:
        q = codes(od)
        assert_codes_close(q[:rows], ref["q"])
        assert np.all(q[rows] == 0x7F), "guard row written"
        if fp8 == "dynamic":
            sc = sd.cpu().numpy()
            assert_scales_close(sc[:rows], ref["scales"], dtype)
            assert np.isnan(sc[rows])
    else:
        ob = bits(od)
        assert_y_close(ob[:rows], ref["y"], dtype)
        assert np.all(ob[rows] == 0x7FC1), "guard row written"


DS = [1, 3, 8, 24, 100, 512, 1000, 3584, 4096, 6656, 14336, 28672]


@pytest.mark.parametrize("d", DS)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_silu_and_mul(orc, dtype, d):
    run_glu(orc, dtype, _x(dtype, 7 if d > 4096 else 33, d), d)


@pytest.mark.parametrize("d", [1, 24, 1000, 6656, 14336])
@pytest.mark.parametrize("fp8", ["static", "dynamic"])
def test_silu_and_mul_fp8(orc, d, fp8):
    run_glu(orc, "bf16", _x("bf16", 9, d, seed=51), d, fp8=fp8, s=0.05 if fp8 == "static" else None)


@pytest.mark.parametrize("rows", [1, 255, 256, 257, 2049])
def test_row_counts(orc, rows):
    run_glu(orc, "bf16", _x("bf16", rows, 512, seed=52), 512, fp8="dynamic")


def test_padded_rows(orc):
    run_glu(orc, "fp16", _x("fp16", 13, 1000, stride=2048, seed=53), 1000)


def test_extreme_gates(orc):
    """Large negative gates (silu ~ g * e^g, tiny but representable), large
    positive gates (silu = g), zeros."""
    rows, d = 4, 512
    rng = np.random.default_rng(54)
    g = np.concatenate([-rng.uniform(20, 95, (1, d)), rng.uniform(20, 1000, (1, d)),
                        np.zeros((1, d)), rng.standard_normal((1, d))]).astype(np.float32)
    u = rng.uniform(0.5, 2, (rows, d)).astype(np.float32)
    x = W.to_bits(np.concatenate([g, u], axis=1), "bf16")
    run_glu(orc, "bf16", x, d)


# Dynamic e4m3 rows whose outputs leave fp32's range: (gate magnitude,
# gate sign or None for random, up magnitude), magnitudes scale * U(1, 2).
# Values are never zero, so no y is 0 where the scale rounds to zero.
WIDE_GLU_ROWS = [
    (2.0**-131, None, 1.0),          # subnormal gates: outputs near 2^-132
    (2.0**-60, None, 2.0**-60),      # outputs near 2^-121 (448 / max overflows fp32)
    (2.0**66, 1.0, 2.0**66),         # products past 2^128, scale finite
    (2.0**70, 1.0, 2.0**70),         # outputs near 2^141: the scale overflows, codes 0
    (2.0**-131, None, 2.0**-131),    # outputs near 2^-263: the scale rounds to zero
    (1.0, None, 1.0),                # an ordinary row beside them
]


def _wide_glu_rows(d, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for gs, gsign, us in WIDE_GLU_ROWS:
        sign = gsign if gsign is not None else np.where(rng.random(d) < 0.5, -1.0, 1.0)
        g = sign * np.minimum(gs * rng.uniform(1.0, 2.0, d), 2.0**127)
        u = np.where(rng.random(d) < 0.5, -1.0, 1.0) * np.minimum(us * rng.uniform(1.0, 2.0, d),
                                                                  2.0**127)
        rows.append(np.concatenate([g, u]))
    return W.to_bits(np.stack(rows).astype(np.float32), "bf16")


@pytest.mark.parametrize("tile", [None, (1, 2), (2, 2), (8, 1), (16, 1)],
                         ids=["auto", "wpr1", "wpr2", "wpr8", "wpr16"])
def test_dynamic_outputs_out_of_fp32_range(orc, tile):
    """Codes and scales of rows whose outputs silu(g) * u overflow fp32,
    fall far below its normal range, or give a scale that overflows or
    rounds to zero, against the fp64 definition; every tile shape."""
    import residual_add_rmsnorm_amd as arn

    d = 1024
    if tile:
        arn.set_tile(*tile)
    try:
        run_glu(orc, "bf16", _wide_glu_rows(d, 61), d, fp8="dynamic")
        if tile:
            assert f"wpr{tile[0]}/nv{tile[1]}/" in arn.last_plan(), arn.last_plan()
    finally:
        arn.set_tile(0, 0)


def _deep_gate_rows(d, seed):
    """Rows whose gates reach far below -87, where exp(-|g|) is under fp32's
    normal range, with up values large enough to lift silu(g) * u into a
    bf16 output's range: (gate range, log2 up range, share of such
    elements; the rest of the row N(0, 1))."""
    rng = np.random.default_rng(seed)
    spec = [((-100.0, -80.0), (0, 40), 1.0),
            ((-130.0, -100.0), (60, 120), 1.0),
            ((-110.0, -85.0), (20, 100), 0.5),      # lanes mixing both kinds
            ((-88.0, -87.0), (100, 126), 1.0),      # around the subnormal edge
            ((-2.0**20, -130.0), (100, 126), 1.0),  # silu below fp64's range
            ((-110.0, -80.0), (10, 30), 1.0 / 64)]  # a few such gates per row
    rows = []
    for (g0, g1), (u0, u1), share in spec:
        g = rng.standard_normal(d)
        u = rng.standard_normal(d)
        pick = rng.random(d) < share
        g[pick] = rng.uniform(g0, g1, pick.sum())
        u[pick] = np.where(rng.random(pick.sum()) < 0.5, -1.0, 1.0) * 2.0 ** rng.uniform(
            u0, u1, pick.sum())
        rows.append(np.concatenate([g, u]))
    return W.to_bits(np.stack(rows).astype(np.float32), "bf16")


@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
@pytest.mark.parametrize("tile", [None, (1, 2), (8, 1), (16, 1)],
                         ids=["auto", "wpr1", "wpr8", "wpr16"])
def test_deep_negative_gates(orc, fp8, tile):
    """silu(g) * u for gates far below -87, whose exp(-|g|) an fp32
    subnormal would hold with few bits or not at all, times up values up to
    2^126: outputs within one bf16 ulp of the definition (codes within one
    step), every output kind and several tile shapes."""
    import residual_add_rmsnorm_amd as arn

    d = 1000
    if tile:
        arn.set_tile(*tile)
    try:
        run_glu(orc, "bf16", _deep_gate_rows(d, 63), d, fp8=fp8,
                s=2.0**-100 if fp8 == "static" else None)
        if tile:
            assert f"wpr{tile[0]}/nv{tile[1]}/" in arn.last_plan(), arn.last_plan()
    finally:
        arn.set_tile(0, 0)


@pytest.mark.parametrize("s", [2.0**-126, 1e-30, 1e-6, 1.0, 1e30, 3.4e38])
def test_static_scale_range(orc, s):
    """Static e4m3 over the range of normal fp32 scales: saturation at one
    end, codes rounding to zero at the other, on gates and ups of ordinary,
    tiny and large magnitude."""
    rng = np.random.default_rng(62)
    d = 1024
    rows = []
    for sc in (1.0, 2.0**-60, 2.0**40):
        g = np.where(rng.random(d) < 0.5, -1.0, 1.0) * sc * rng.uniform(0.5, 2.0, d)
        u = np.where(rng.random(d) < 0.5, -1.0, 1.0) * sc * rng.uniform(0.5, 2.0, d)
        rows.append(np.concatenate([g, u]))
    x = W.to_bits(np.stack(rows).astype(np.float32), "bf16")
    run_glu(orc, "bf16", x, d, fp8="static", s=s)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_nonfinite_inputs_propagate(orc, dtype):
    """Infinities and NaNs follow IEEE arithmetic through g / (1 + exp(-g))
    * u: silu(+inf) = inf, silu(-inf) = -inf / inf = NaN, 0 * inf = NaN, a
    finite nonzero silu times an infinite up is infinite, NaN anywhere gives
    NaN; other elements of the row are unaffected.  16-bit outputs (e4m3
    codes of non-finite y are not specified)."""
    d = 300
    inf, nan = (0x7F80, 0x7FC0) if dtype == "bf16" else (0x7C00, 0x7E00)
    one, two, mfive = (0x3F80, 0x4000, 0xC0A0) if dtype == "bf16" else (0x3C00, 0x4000, 0xC500)
    x = _x(dtype, 2, d, seed=57)
    cases = [(inf, two), (inf | 0x8000, two), (nan, two), (one, inf), (0, inf),
             (mfive, inf | 0x8000), (two, nan), (0x8000, inf | 0x8000)]
    for j, (g, u) in enumerate(cases):
        x[0, 7 * j] = g
        x[0, d + 7 * j] = u
    x[1, 2 * d - 1] = inf  # the last up value of a row
    run_glu(orc, dtype, x, d)


def test_zero_row_dynamic(orc):
    x = _x("bf16", 5, 768, seed=55)
    x[2] = 0
    run_glu(orc, "bf16", x, 768, fp8="dynamic")


def test_split_gate_and_up_tensors(orc):
    """The C ABI with gate and up in separate tensors of different strides."""
    from residual_add_rmsnorm_amd import _lib

    lib = _lib.load()
    rows, d = 20, 1024
    g = _x("bf16", rows, d // 2, seed=56)[:, :d]      # (rows, d) values
    u = _x("bf16", rows, d // 2, seed=57)[:, :d]
    gate = np.full((rows, 1536), W.PAD_SENTINEL, np.uint16)
    up = np.full((rows, 1280), W.PAD_SENTINEL, np.uint16)
    gate[:, :d], up[:, :d] = g, u
    gd, ud = dev(gate, "bf16"), dev(up, "bf16")
    out = torch.empty(rows, d, dtype=torch.bfloat16, device="cuda")
    st = lib.arn_silu_and_mul(out.data_ptr(), d, gd.data_ptr(), 1536, ud.data_ptr(), 1280, rows, d,
                              _lib.BF16, torch.cuda.current_stream().cuda_stream)
    assert st == _lib.OK
    torch.cuda.synchronize()
    ref = orc.silu_and_mul_split("bf16", gate, up, d=d)
    assert_y_close(bits(out), ref["y"], "bf16")


@pytest.mark.parametrize("wpr,nv", [(1, 2), (1, 4), (2, 2), (2, 4), (4, 1), (4, 2), (4, 4), (8, 1),
                                    (8, 2), (8, 4), (16, 1), (16, 2), (16, 4), (16, 8)])
def test_forced_tiles(orc, wpr, nv):
    import residual_add_rmsnorm_amd as arn

    d = 64 * wpr * nv * 8 - 24
    arn.set_tile(wpr, nv)
    try:
        run_glu(orc, "bf16", _x("bf16", 5, d, seed=58), d, fp8="dynamic")
        assert f"wpr{wpr}/nv{nv}/" in arn.last_plan(), arn.last_plan()
    finally:
        arn.set_tile(0, 0)


@pytest.mark.parametrize("d,tile", [(1024, "wpr1/nv2/rpb4"), (1792, "wpr2/nv2/rpb2"),
                                    (3584, "wpr4/nv2/rpb1"), (4096, "wpr4/nv2/rpb1"),
                                    (6656, "wpr8/nv2/rpb1")])
@pytest.mark.parametrize("fp8", [None, "dynamic", "static"])
def test_many_rows_automatic_tiles(orc, d, tile, fp8):
    """With many rows (at least 4 per CU) rows up to 4096 wide take the
    fewest waves whose lanes hold at most two vectors; wider rows keep
    eight-wave rows.  Every row of 4 x CUs + 3 rows against the oracle."""
    import residual_add_rmsnorm_amd as arn

    rows = 4 * torch.cuda.get_device_properties(0).multi_processor_count + 3
    run_glu(orc, "bf16", _x("bf16", rows, d, seed=60 + d % 89), d, fp8=fp8,
            s=0.05 if fp8 == "static" else None)
    assert f"/vec8/{tile}/" in arn.last_plan(), arn.last_plan()


@pytest.mark.parametrize("name", ["silu_and_mul_fp8_dynamic_bf16_32768x6656",
                                  "silu_and_mul_fp8_static_bf16_decode_x6656"])
def test_workloads_sampled(orc, name):
    """Full-size workloads in the benchmark's launch configuration; sampled
    rows against the oracle."""
    import residual_add_rmsnorm_amd as arn

    w = W.WORKLOADS[name]
    d_in = W.make(w)
    x = dev(d_in["x"], w.dtype)
    out = torch.full((w.rows, w.hidden), 0x7F, dtype=torch.uint8, device="cuda")
    ov = out.view(torch.float8_e4m3fn)
    if w.fp8 == "dynamic":
        sc = torch.empty(w.rows, dtype=torch.float32, device="cuda")
        arn.silu_and_mul_fp8(x, dynamic=True, out=ov, scales_out=sc)
        s = 0.0
    else:
        s = static_scale(name)
        sc = torch.tensor([s], dtype=torch.float32, device="cuda")
        arn.silu_and_mul_fp8(x, scale=sc, out=ov)
    torch.cuda.synchronize()
    idx = np.unique(np.linspace(0, w.rows - 1, 96).astype(np.int64))
    mode = O.FP8_DYNAMIC if w.fp8 == "dynamic" else O.FP8_STATIC
    ref = orc.silu_and_mul(w.dtype, d_in["x"][idx], d=w.hidden, fp8_mode=mode, static_scale=s)
    assert_codes_close(codes(out)[idx], ref["q"])
    if w.fp8 == "dynamic":
        assert_scales_close(sc.cpu().numpy()[idx], ref["scales"], w.dtype)


def test_rows_past_4gib_and_launch_split(orc):
    """A gate|up tensor of 8 GiB and more rows than one launch takes: with
    the one-row-per-block tile forced, 2^22 rows fill a launch, so 2^22 +
    1000 rows of d = 512 take two, the second starting 8 GiB into the input
    and 2 GiB into the codes; dynamic e4m3, so the per-row scales are offset
    too.  Sampled rows on both sides of the boundary against the oracle."""
    import residual_add_rmsnorm_amd as arn

    rows, d = (1 << 22) + 1000, 512
    print(f"\n[past-4GiB] silu_and_mul_fp8 rows {rows} d {d}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4343)
    x = device_normal(rows, 2 * d, 2.0, gen)
    b = 1 << 22
    idx = np.unique(np.concatenate([np.linspace(0, rows - 1, 64).astype(np.int64),
                                    np.arange(b - 3, b + 3), np.arange(rows - 3, rows)]))
    sel = torch.from_numpy(idx).cuda()
    xs = bits(x.index_select(0, sel))
    out = torch.full((rows, d), 0x7F, dtype=torch.uint8, device="cuda")
    sc = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    arn.set_tile(8, 1)
    try:
        arn.silu_and_mul_fp8(x, dynamic=True, out=out.view(torch.float8_e4m3fn), scales_out=sc)
        plan = arn.last_plan()
    finally:
        arn.set_tile(0, 0)
    torch.cuda.synchronize()
    print(f"[past-4GiB] plan {plan}", flush=True)
    assert plan.endswith("wpr8/nv1/rpb1/grid1000")
    ref = orc.silu_and_mul("bf16", xs, d=d, fp8_mode=O.FP8_DYNAMIC)
    assert_codes_close(codes(out.index_select(0, sel)), ref["q"])
    assert_scales_close(sc.index_select(0, sel).cpu().numpy(), ref["scales"], "bf16")
    assert not bool(torch.isnan(sc).any()), "a row's scale was not written"
    for i in range(0, rows, 1 << 20):
        j = min(rows, i + (1 << 20))
        assert not bool(((out[i:j] & 0x7F) == 0x7F).any()), f"unwritten codes in rows {i}..{j}"
