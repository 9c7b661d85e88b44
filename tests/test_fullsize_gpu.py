"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (automatic kernel shape, dense or strided rows as given).

The oracle computes sampled rows one by one (the generator is keyed per
block of rows, so any row can be regenerated); properties that hold at any
size are checked over every row: the stored residual equals the fp32 sum of
its inputs rounded to 16 bits (the double-rounding rule the oracle's pins
establish) and no byte of row padding changes.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import (TORCH_DT, assert_codes_close, assert_scales_close, assert_y_close,
                            bits, codes, dev, device_normal, static_scale)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _sample_rows(rows, n=160):
    idx = np.unique(np.concatenate([np.linspace(0, rows - 1, n).astype(np.int64),
                                    [0, 1, rows // 2, rows - 2, rows - 1]]))
    return idx[(idx >= 0) & (idx < rows)]


@pytest.mark.parametrize("name", [
    "rmsnorm_bf16_64x4096",
    "fused_add_rmsnorm_bf16_4096x8192",
    "fused_add_rmsnorm_fp8_static_fp16_decode_x16384",
    "fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168",
    "fused_add_rmsnorm_bf16_65536x3840_stride4096",
    "fused_add_rmsnorm_bf16_65536x2880_stride4096",
])
def test_full_size(orc, name):
    import residual_add_rmsnorm_amd as arn

    w = W.WORKLOADS[name]
    print(f"\n[full-size] {name}", flush=True)
    d = W.make(w)
    rows, H, S = w.rows, w.hidden, w.stride
    dt = TORCH_DT[w.dtype]
    x = dev(d["x"], w.dtype)
    wd = dev(d["weight"], w.dtype)
    res = dev(d["residual"], w.dtype) if w.has_residual else None
    xv = x[:, :H]
    rv = res[:, :H] if res is not None else None

    if w.fp8:
        out = torch.full((rows, S), 0x7F, dtype=torch.uint8, device="cuda")
        ov = out.view(torch.float8_e4m3fn)[:, :H]
        if w.fp8 == "static":
            s = static_scale()
            sc = torch.tensor([s], dtype=torch.float32, device="cuda")
            arn.fused_add_rmsnorm_fp8(xv, rv, wd, w.eps, scale=sc, out=ov)
        else:
            s = 0.0
            sc = torch.empty(rows, dtype=torch.float32, device="cuda")
            arn.fused_add_rmsnorm_fp8(xv, rv, wd, w.eps, dynamic=True, out=ov, scales_out=sc)
    else:
        out = torch.full((rows, S), float("nan"), dtype=dt, device="cuda")
        ov = out[:, :H]
        if rv is not None:
            arn.fused_add_rmsnorm(xv, rv, wd, w.eps, out=ov)
        else:
            arn.rmsnorm(xv, wd, w.eps, out=ov)
    torch.cuda.synchronize()
    print(f"[full-size] plan {arn.last_plan()}", flush=True)

    # every row: stored residual = RNE16(fp32(x) + fp32(residual)); padding intact
    if res is not None:
        x0 = torch.from_numpy(d["x"].view(np.int16)).view(dt)
        r0 = torch.from_numpy(d["residual"].view(np.int16)).view(dt)
        expect = (x0[:, :H].float() + r0[:, :H].float()).to(dt)
        got = res.cpu()
        assert torch.equal(got[:, :H].view(torch.int16), expect.view(torch.int16))
        if S > H:
            assert bool((got[:, H:].view(torch.int16) == W.PAD_SENTINEL).all())
            assert bool((x.cpu()[:, H:].view(torch.int16) == W.PAD_SENTINEL).all())
    if S > H:
        pad = out[:, H:].cpu()
        if w.fp8:
            assert bool((pad == 0x7F).all())
        else:
            assert bool(torch.isnan(pad.float()).all())

    # sampled rows against the oracle
    idx = _sample_rows(rows)
    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[w.fp8]
    ref = orc.add_rmsnorm(w.dtype, d["x"][idx], d["residual"][idx] if res is not None else None,
                          d["weight"], w.eps, hidden=H, fp8_mode=mode, static_scale=s if w.fp8 else 0.0)
    if res is not None:
        assert np.array_equal(bits(res[idx.tolist()])[:, :H], ref["r16"])
    if w.fp8:
        assert_codes_close(codes(out[idx.tolist()])[:, :H], ref["q"])
        if w.fp8 == "dynamic":
            assert_scales_close(sc.cpu().numpy()[idx], ref["scales"], w.dtype)
    else:
        assert_y_close(bits(out[idx.tolist()])[:, :H], ref["y"], w.dtype)



@pytest.mark.parametrize("fp8", [None, "dynamic"])
def test_rows_past_4gib_and_launch_split(orc, fp8):
    """Tensors larger than 4 GiB, and more rows than one launch takes: with
    the one-row-per-block tile forced (8 waves, one vector per lane), 2^22
    rows fill one launch, so 2^22 + 1000 rows of 512 bf16 take two launches,
    the second starting exactly 4 GiB into each tensor.  Inputs are drawn on
    the device (seeded); the oracle checks rows on both sides of the launch
    boundary and spread over the whole range, and the stored residual is
    checked over every row against the fp32 sum rounded to bf16."""
    import residual_add_rmsnorm_amd as arn

    rows, H, eps = (1 << 22) + 1000, 512, 1e-6
    assert rows * H * 2 > 1 << 32
    print(f"\n[past-4GiB] rows {rows} hidden {H} fp8 {fp8}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    chunk = 1 << 20
    x = device_normal(rows, H, 1.0, gen)
    res = device_normal(rows, H, 1.0, gen)
    res0 = res.clone()
    w = (1 + 0.1 * torch.randn(H, generator=gen, device="cuda")).to(torch.bfloat16)
    b = 1 << 22
    idx = np.unique(np.concatenate([_sample_rows(rows, 64), np.arange(b - 3, b + 3),
                                    np.arange(rows - 3, rows)]))
    sel = torch.from_numpy(idx).cuda()
    xs, rs = bits(x.index_select(0, sel)), bits(res.index_select(0, sel))

    arn.set_tile(8, 1)
    try:
        if fp8:
            out = torch.full((rows, H), 0x7F, dtype=torch.uint8, device="cuda")
            sc = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
            arn.fused_add_rmsnorm_fp8(x, res, w, eps, dynamic=True,
                                      out=out.view(torch.float8_e4m3fn), scales_out=sc)
        else:
            out = torch.full((rows, H), float("nan"), dtype=torch.bfloat16, device="cuda")
            arn.fused_add_rmsnorm(x, res, w, eps, out=out)
        plan = arn.last_plan()
    finally:
        arn.set_tile(0, 0)
    torch.cuda.synchronize()
    print(f"[past-4GiB] plan {plan}", flush=True)
    assert plan.endswith("wpr8/nv1/rpb1/grid1000")  # the last launch: the rows past 2^22

    for i in range(0, rows, chunk):
        j = min(rows, i + chunk)
        expect = (x[i:j].float() + res0[i:j].float()).to(torch.bfloat16)
        assert torch.equal(res[i:j].view(torch.int16), expect.view(torch.int16)), f"rows {i}..{j}"
    del res0

    mode = O.FP8_DYNAMIC if fp8 else O.FP8_NONE
    ref = orc.add_rmsnorm("bf16", xs, rs, bits(w), eps, hidden=H, fp8_mode=mode)
    assert np.array_equal(bits(res.index_select(0, sel)), ref["r16"])
    if fp8:
        assert_codes_close(codes(out.index_select(0, sel)), ref["q"])
        assert_scales_close(sc.index_select(0, sel).cpu().numpy(), ref["scales"], "bf16")
        assert not bool(torch.isnan(sc).any()), "a row's scale was not written"
    else:
        assert_y_close(bits(out.index_select(0, sel)), ref["y"], "bf16")
    # every output written (the canaries are NaN codes / NaNs; the outputs are finite)
    for i in range(0, rows, chunk):
        j = min(rows, i + chunk)
        o = out[i:j]
        bad = ((o & 0x7F) == 0x7F).any() if fp8 else torch.isnan(o.float()).any()
        assert not bool(bad), f"unwritten output in rows {i}..{j}"
