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
                            bits, codes, dev, static_scale)

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
