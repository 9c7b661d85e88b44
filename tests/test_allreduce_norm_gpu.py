"""Parity of the all-reduce form (arn_sum_add_rmsnorm): the partial rows of
nparts ranks summed in fp32 in rank order and rounded once to 16 bits, then
the fused residual add + RMSNorm (+ e4m3), against the oracle's
sum_add_rmsnorm (its all-reduce step composed with add_rmsnorm).

Comparison rules as for the norm: stored residual bit-exact, y within
max(rho |y|, ulp16), codes within one e4m3 step, dynamic scales within rho;
row padding, guard rows and the parts themselves unchanged."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import (assert_codes_close, assert_scales_close, assert_y_close,
                            bits, codes, dev, device_normal)

pytestmark = pytest.mark.gpu

CANARY16 = 0x7FC1
CANARY8 = 0x7F


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _random(dtype, rows, hidden, stride, seed, std=1.0):
    rng = np.random.default_rng(seed)
    a = np.full((rows, stride), W.PAD_SENTINEL, np.uint16)
    a[:, :hidden] = W.to_bits((rng.standard_normal((rows, hidden)) * std).astype(np.float32), dtype)
    return a


def run_case(orc, *, dtype, parts, res, w, eps, hidden, fp8=None, s=None, alias_out=False):
    import residual_add_rmsnorm_amd as arn

    rows, stride = parts[0].shape
    fused = res is not None

    def with_guard(a):
        g = np.full((rows + 1, a.shape[1]), W.PAD_SENTINEL, np.uint16)
        g[:rows] = a
        return g

    pd = [dev(with_guard(p), dtype) for p in parts]
    pv = [p[:rows, :hidden] for p in pd]
    rd = dev(with_guard(res), dtype) if fused else None
    rv = rd[:rows, :hidden] if fused else None
    wd = dev(w, dtype) if w is not None else None
    kw = {}
    if fp8:
        od = torch.full((rows + 1, stride), CANARY8, dtype=torch.uint8, device="cuda")
        ov = od.view(torch.float8_e4m3fn)[:rows, :hidden]
        if fp8 == "static":
            kw = dict(fp8="static", scale=torch.tensor([s], dtype=torch.float32, device="cuda"))
        else:
            sd = torch.full((rows + 1,), float("nan"), dtype=torch.float32, device="cuda")
            kw = dict(fp8="dynamic", scales_out=sd[:rows])
    elif alias_out:
        od, ov = pd[0], pv[0]
    else:
        od = dev(np.full((rows + 1, stride), CANARY16, np.uint16), dtype)
        ov = od[:rows, :hidden]
    arn.sum_add_rmsnorm(pv, wd, eps, residual=rv, out=ov, **kw)
    torch.cuda.synchronize()

    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.sum_add_rmsnorm(dtype, parts, res, w, eps, hidden=hidden, fp8_mode=mode,
                              static_scale=s or 0.0)
    if fused:
        rb = bits(rd)
        assert np.array_equal(rb[:rows, :hidden], ref["r16"]), "stored residual not bit-exact"
        assert np.all(rb[:rows, hidden:] == W.PAD_SENTINEL), "residual padding written"
        assert np.all(rb[rows] == W.PAD_SENTINEL), "residual guard row written"
    for g, p in enumerate(pd):
        if alias_out and g == 0:
            continue
        assert np.array_equal(bits(p)[:rows], parts[g]), f"part {g} modified"
    if fp8:
        q = codes(od)
        assert_codes_close(q[:rows, :hidden], ref["q"])
        assert np.all(q[:rows, hidden:] == CANARY8) and np.all(q[rows] == CANARY8)
        if fp8 == "dynamic":
            sc = sd.cpu().numpy()
            assert_scales_close(sc[:rows], ref["scales"], dtype)
            assert np.isnan(sc[rows])
    else:
        ob = bits(od)
        assert_y_close(ob[:rows, :hidden], ref["y"], dtype)
        if not alias_out:
            assert np.all(ob[:rows, hidden:] == CANARY16) and np.all(ob[rows] == CANARY16)
    return arn.last_plan()


@pytest.mark.parametrize("nparts", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
@pytest.mark.parametrize("fused", [True, False])
def test_parts_and_modes(orc, nparts, fp8, fused):
    dtype = "bf16" if nparts % 2 else "fp16"
    rows, hidden = 37, 4096
    parts = [_random(dtype, rows, hidden, hidden, 10 + g, std=nparts ** -0.5)
             for g in range(nparts)]
    res = _random(dtype, rows, hidden, hidden, 9) if fused else None
    w = _random(dtype, 1, hidden, hidden, 8)[0]
    plan = run_case(orc, dtype=dtype, parts=parts, res=res, w=w, eps=1e-6, hidden=hidden,
                    fp8=fp8, s=0.01 if fp8 == "static" else None)
    assert plan.startswith("sum_")


@pytest.mark.parametrize("hidden,stride", [(1, 1), (7, 7), (100, 104), (513, 520), (2880, 4096),
                                           (7168, 7168), (8192, 8192), (16384, 16384),
                                           (32768, 32768), (999, 1001)])
def test_hidden_sweep(orc, hidden, stride):
    rows = 3 if hidden > 8192 else 19
    parts = [_random("bf16", rows, hidden, stride, 20 + g, std=0.5) for g in range(4)]
    res = _random("bf16", rows, hidden, stride, 19)
    w = _random("bf16", 1, hidden, hidden, 18)[0]
    run_case(orc, dtype="bf16", parts=parts, res=res, w=w, eps=1e-5, hidden=hidden)


@pytest.mark.parametrize("nparts,hidden,tile", [(2, 4096, "wpr4/nv2/"), (3, 4096, "wpr4/nv2/"),
                                                (2, 6144, "wpr8/nv2/"), (8, 4096, "wpr8/nv1/")])
def test_many_rows_automatic_tiles(orc, nparts, hidden, tile):
    """With many rows, two or three parts take the compact tile up to two
    vectors per lane; four or more parts keep one vector per lane with more
    waves.  4 x CUs + 2 rows, every row against the oracle."""
    rows = 4 * torch.cuda.get_device_properties(0).multi_processor_count + 2
    parts = [_random("bf16", rows, hidden, hidden, 50 + g, std=nparts ** -0.5)
             for g in range(nparts)]
    res = _random("bf16", rows, hidden, hidden, 49)
    w = _random("bf16", 1, hidden, hidden, 48)[0]
    plan = run_case(orc, dtype="bf16", parts=parts, res=res, w=w, eps=1e-6, hidden=hidden)
    assert f"/vec8/{tile}" in plan, plan


@pytest.mark.parametrize("rows", [1, 255, 1029])
def test_row_counts(orc, rows):
    parts = [_random("fp16", rows, 1024, 1024, 30 + g) for g in range(3)]
    res = _random("fp16", rows, 1024, 1024, 29, std=2.0)
    run_case(orc, dtype="fp16", parts=parts, res=res, w=None, eps=1e-6, hidden=1024)


def test_rank_order_is_followed():
    """2^24 + 1 rounds back to 2^24 in fp32: parts (2^24, 1, -2^24) reduce to
    0 and (2^24, -2^24, 1) to 1.  With a zero residual the stored residual
    is the reduced value itself."""
    import residual_add_rmsnorm_amd as arn

    vals = {"a": 0x4B80, "one": 0x3F80, "b": 0xCB80}
    for order, expect in ((("a", "one", "b"), 0x0000), (("a", "b", "one"), 0x3F80)):
        parts = [torch.full((2, 64), 0, dtype=torch.int16, device="cuda") for _ in order]
        for p, k in zip(parts, order):
            p.fill_(int(np.uint16(vals[k]).view(np.int16)))
        pv = [p.view(torch.bfloat16) for p in parts]
        res = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
        arn.sum_add_rmsnorm(pv, None, 1e-6, residual=res)
        torch.cuda.synchronize()
        assert np.all(bits(res) == expect), (order, bits(res)[0, :4])


def test_out_aliases_first_part(orc):
    parts = [_random("bf16", 9, 2048, 2048, 40 + g) for g in range(2)]
    res = _random("bf16", 9, 2048, 2048, 39)
    run_case(orc, dtype="bf16", parts=parts, res=res, w=None, eps=1e-6, hidden=2048,
             alias_out=True)


@pytest.mark.parametrize("hidden,served", [
    (32768, True), (32776, False),   # 128-bit accesses: 16 waves x 4 vectors x 8
    (16380, True), (16388, False),   # hidden % 8 == 4: 64-bit accesses, x 4
    (8190, True), (8194, False),     # hidden % 4 == 2: 32-bit accesses, x 2
    (4095, True), (4097, False),     # odd: 16-bit accesses
])
def test_largest_rows(orc, hidden, served):
    import residual_add_rmsnorm_amd as arn

    parts = [_random("bf16", 2, hidden, hidden, 50 + g) for g in range(2)]
    res = _random("bf16", 2, hidden, hidden, 49)
    if served:
        run_case(orc, dtype="bf16", parts=parts, res=res, w=None, eps=1e-6, hidden=hidden)
        return
    with pytest.raises(arn.ArnError) as e:
        arn.sum_add_rmsnorm([dev(p, "bf16") for p in parts], None, 1e-6,
                            residual=dev(res, "bf16"))
    assert e.value.status == 2


def test_refusals():
    import residual_add_rmsnorm_amd as arn

    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        arn.sum_add_rmsnorm([x] * 9, None, 1e-6)                   # too many parts
    with pytest.raises(ValueError):
        arn.sum_add_rmsnorm([x, torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda")],
                            None, 1e-6)                             # shape mismatch
    with pytest.raises(arn.ArnError) as e:
        arn.sum_add_rmsnorm([x, x.clone()], None, 1e-6, residual=x)  # residual aliases a part
    assert e.value.status == 1


def test_full_size(orc):
    """The benchmark's workload (8 ranks x 4096 x 8192 bf16) in its launch
    configuration: sampled rows against the oracle; the stored residual of
    every row against the oracle's reduction + fp32 add rule."""
    import residual_add_rmsnorm_amd as arn

    w = W.WORKLOADS["sum_add_rmsnorm_bf16_8x4096x8192"]
    print(f"\n[full-size] {w.name}", flush=True)
    d = W.make(w)
    pd = [dev(p, w.dtype) for p in d["parts"]]
    rd = dev(d["residual"], w.dtype)
    wd = dev(d["weight"], w.dtype)
    y = arn.sum_add_rmsnorm(pd, wd, w.eps, residual=rd)
    torch.cuda.synchronize()
    idx = np.unique(np.concatenate([np.linspace(0, w.rows - 1, 96).astype(np.int64),
                                    [0, 1, w.rows - 1]]))
    ref = orc.sum_add_rmsnorm(w.dtype, [p[idx] for p in d["parts"]], d["residual"][idx],
                              d["weight"], w.eps)
    rb, yb = bits(rd), bits(y)
    assert np.array_equal(rb[idx], ref["r16"])
    assert_y_close(yb[idx], ref["y"], w.dtype)
    # every row's stored residual: the oracle's reduction, then the fp32 add
    # rounded once (pinned exhaustively against the oracle's residual step)
    x16 = orc.sum_parts(w.dtype, d["parts"])
    xf = torch.from_numpy(x16.view(np.int16)).view(torch.bfloat16).float()
    r0 = torch.from_numpy(d["residual"].view(np.int16)).view(torch.bfloat16).float()
    expect = (xf + r0).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rb, expect)


def test_rows_past_4gib_and_launch_split(orc):
    """Parts, residual and output of 4 GiB and more, and more rows than one
    launch takes (the one-row-per-block tile forced: 2^22 rows per launch),
    so every part's pointer of the second launch starts 4 GiB in.  Two parts,
    fused residual, 16-bit output; sampled rows on both sides of the launch
    boundary against the oracle."""
    import residual_add_rmsnorm_amd as arn

    rows, H, eps = (1 << 22) + 1000, 512, 1e-6
    print(f"\n[past-4GiB] sum_add_rmsnorm 2 parts rows {rows} hidden {H}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4444)
    parts = [device_normal(rows, H, 0.7, gen) for _ in range(2)]
    res = device_normal(rows, H, 1.0, gen)
    w = (1 + 0.1 * torch.randn(H, generator=gen, device="cuda")).to(torch.bfloat16)
    b = 1 << 22
    idx = np.unique(np.concatenate([np.linspace(0, rows - 1, 64).astype(np.int64),
                                    np.arange(b - 3, b + 3), np.arange(rows - 3, rows)]))
    sel = torch.from_numpy(idx).cuda()
    ps = [bits(p.index_select(0, sel)) for p in parts]
    rs = bits(res.index_select(0, sel))
    out = torch.full((rows, H), float("nan"), dtype=torch.bfloat16, device="cuda")
    arn.set_tile(8, 1)
    try:
        arn.sum_add_rmsnorm(parts, w, eps, residual=res, out=out)
        plan = arn.last_plan()
    finally:
        arn.set_tile(0, 0)
    torch.cuda.synchronize()
    print(f"[past-4GiB] plan {plan}", flush=True)
    assert plan.endswith("wpr8/nv1/rpb1/grid1000")
    ref = orc.sum_add_rmsnorm("bf16", ps, rs, bits(w), eps)
    assert np.array_equal(bits(res.index_select(0, sel)), ref["r16"])
    assert_y_close(bits(out.index_select(0, sel)), ref["y"], "bf16")
    for i in range(0, rows, 1 << 20):
        j = min(rows, i + (1 << 20))
        assert not bool(torch.isnan(out[i:j].float()).any()), f"unwritten output in rows {i}..{j}"
