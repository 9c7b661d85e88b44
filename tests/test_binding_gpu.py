"""The binding's native marshalling on GPU tensors: each refused argument
raises ValueError before anything is launched (outputs and residual keep
their bytes), a status from the C ABI comes back as ArnError, and outputs
the binding allocates have the documented shapes and dtypes."""
import pytest
import torch

import residual_add_rmsnorm_amd as arn

pytestmark = pytest.mark.gpu

E4M3 = torch.float8_e4m3fn


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _t(*shape, dtype=torch.bfloat16, fill=1.0):
    return torch.full(shape, fill, dtype=dtype, device="cuda")


def _refused(call, match):
    with pytest.raises(ValueError, match=match):
        call()


def test_norm_refusals_launch_nothing():
    x = _t(4, 64)
    res = _t(4, 64, fill=2.0)
    w = _t(64)
    out = _t(4, 64, fill=7.0)
    codes = torch.full((4, 64), 0x55, dtype=torch.uint8, device="cuda").view(E4M3)
    s = torch.ones(1, device="cuda")
    cases = [
        (lambda: arn.rmsnorm(x.float(), None, 1e-6), "bfloat16 or float16"),
        (lambda: arn.rmsnorm(x, w.half(), 1e-6, out=out), "weight dtype"),
        (lambda: arn.rmsnorm(x, _t(63), 1e-6, out=out), "contiguous vector of 64"),
        (lambda: arn.rmsnorm(x, _t(128)[::2], 1e-6, out=out), "contiguous vector of 64"),
        (lambda: arn.rmsnorm(x, w, 1e-6, out=_t(4, 32)), "x's shape"),
        (lambda: arn.rmsnorm(x, w, 1e-6, out=out.half()), "x's shape"),
        (lambda: arn.fused_add_rmsnorm(x, res.half(), w, 1e-6, out=out), "residual must match"),
        (lambda: arn.fused_add_rmsnorm(x, _t(4, 32), w, 1e-6, out=out), "residual must match"),
        (lambda: arn.fused_add_rmsnorm(x, res.t().contiguous().t(), w, 1e-6, out=out),
         "unit stride"),
        (lambda: arn.fused_add_rmsnorm_fp8(x, res, w, 1e-6, out=codes), "needs `scale`"),
        (lambda: arn.fused_add_rmsnorm_fp8(x, res, w, 1e-6, scale=s.double(), out=codes),
         "one float32 value"),
        (lambda: arn.fused_add_rmsnorm_fp8(x, res, w, 1e-6, scale=torch.ones(2, device="cuda"),
                                           out=codes), "one float32 value"),
        (lambda: arn.fused_add_rmsnorm_fp8(x, res, w, 1e-6, dynamic=True, out=codes,
                                           scales_out=torch.ones(3, device="cuda")),
         "4 contiguous float32"),
        (lambda: arn.rmsnorm_fp8(x, w, 1e-6, scale=s, out=out), "x's shape and dtype"),
        (lambda: arn.norm(x, w, 1e-6, fp8="fnuz", out=codes, scale=s), "fp8 must be"),
        (lambda: arn.norm(x, w, 1e-6, residual=_t(2, 64), out=out), "residual must match"),
    ]
    for call, match in cases:
        _refused(call, match)
    torch.cuda.synchronize()
    assert bool((res == 2.0).all()) and bool((out == 7.0).all())
    assert bool((codes.view(torch.uint8) == 0x55).all())


def test_glu_and_gemm_refusals():
    g = _t(4, 130)
    _refused(lambda: arn.silu_and_mul(_t(4, 65)), "2\\*d")
    _refused(lambda: arn.silu_and_mul(g, out=_t(4, 64)), "shape \\(4, 65\\)")
    _refused(lambda: arn.silu_and_mul_fp8(g, scale=None), "needs `scale`")
    a = torch.zeros(2, 256, dtype=torch.uint8, device="cuda")
    b = torch.zeros(32, 256, dtype=torch.uint8, device="cuda")
    s1 = torch.ones(1, device="cuda")
    _refused(lambda: arn.fp8_gemm(a.float(), s1, b, s1), "2-D e4m3")
    _refused(lambda: arn.fp8_gemm(a, s1, b[:, :128], s1), "same K")
    _refused(lambda: arn.fp8_gemm(a, torch.ones(3, device="cuda"), b, s1), "scale_a must hold 1 or 2")
    _refused(lambda: arn.fp8_gemm(a, s1, b, s1, out_dtype=torch.float32), "out must be")
    _refused(lambda: arn.fp8_gemm(a, s1, b, s1, out=_t(2, 31)), "out must be")
    ws = torch.zeros(64, 2, dtype=torch.uint8, device="cuda").t()
    _refused(lambda: arn.fp8_gemm(a, s1, b, s1, workspace=ws), "workspace must be")
    _refused(lambda: arn.fp8_gemm_preshuffled_noalloc(a, s1, b, s1), "PreshuffledWeight")


def test_abi_status_becomes_arn_error():
    # 65537 elements with a 2-byte aligned row: valid, but above the largest
    # row served at that alignment, so the C ABI answers ARN_EUNSUPPORTED.
    x = torch.zeros(1, 65537, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(arn.ArnError) as e:
        arn.rmsnorm(x, None, 1e-6)
    assert e.value.status == 2 and "arn_rmsnorm" in str(e.value)


def test_allocated_outputs():
    x = _t(2, 3, 64)
    res = _t(2, 3, 64)
    q, s = arn.fused_add_rmsnorm_fp8(x, res, None, 1e-6, dynamic=True)
    assert q.shape == (2, 3, 64) and q.dtype == E4M3 and s.shape == (2, 3) and s.dtype == torch.float32
    q1, s1 = arn.rmsnorm_fp8(_t(64), None, 1e-6, dynamic=True)
    assert q1.shape == (64,) and s1.shape == (1,)
    y = arn.norm(x, None, 1e-6, variance_size=32)
    assert y.shape == x.shape and y.dtype == x.dtype
    o = arn.silu_and_mul(_t(5, 2, 128, dtype=torch.float16))
    assert o.shape == (5, 2, 64) and o.dtype == torch.float16
    c = arn.fp8_gemm(torch.zeros(3, 128, dtype=torch.uint8, device="cuda"),
                     torch.ones(1, device="cuda"),
                     torch.zeros(16, 128, dtype=torch.uint8, device="cuda"),
                     torch.ones(1, device="cuda"), out_dtype=torch.float16)
    assert c.shape == (3, 16) and c.dtype == torch.float16
    torch.cuda.synchronize()
    assert bool((c == 0).all())


def test_torch_ops_refusals_and_status():
    import residual_add_rmsnorm_amd.torch_ops  # noqa: F401  (registers arn::*)

    x = torch.zeros(1, 65537, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="arn_rmsnorm.*status 2"):
        torch.ops.arn.rmsnorm(x, None, 1e-6)
    with pytest.raises(ValueError, match="bfloat16 or float16"):
        torch.ops.arn.rmsnorm(x.float(), None, 1e-6)
    g = _t(2, 64)
    with pytest.raises(ValueError, match="one float32 value"):
        torch.ops.arn.silu_and_mul_fp8_static(g, torch.ones(2, device="cuda"))
    a = torch.zeros(1, 256, dtype=torch.uint8, device="cuda")
    s1 = torch.ones(1, device="cuda")
    small = torch.zeros(2048, dtype=torch.uint8, device="cuda")  # one of the weight's two 16 x 128 tiles
    with pytest.raises(ValueError, match="smaller than a pre-shuffled"):
        torch.ops.arn.fp8_gemm_preshuffled(a, s1, small, 16, 256, s1)
    c = torch.ops.arn.fp8_gemm_preshuffled(a, s1, torch.zeros(4096, dtype=torch.uint8,
                                                              device="cuda"), 16, 256, s1)
    torch.cuda.synchronize()
    assert c.shape == (1, 16) and c.dtype == torch.bfloat16 and bool((c == 0).all())


@pytest.mark.parametrize("dtype,rows,hidden,fused,fp8", [
    ("fp16", 1, 16384, True, "static"), ("bf16", 256, 8192, True, None),
    ("fp16", 384, 7168, True, "dynamic"), ("fp16", 100, 5120, True, None),
    ("bf16", 1030, 1024, False, "dynamic"), ("bf16", 64, 4096, False, None),
    ("bf16", 4100, 3840, True, None)])
def test_plan_query_matches_the_launch(dtype, rows, hidden, fused, fp8):
    """arn_norm_plan, given this device's CU count, names the kernel the
    call then launches (arn_last_plan)."""
    td = torch.bfloat16 if dtype == "bf16" else torch.float16
    x = torch.randn(rows, hidden, device="cuda").to(td)
    res = torch.randn(rows, hidden, device="cuda").to(td) if fused else None
    w = torch.ones(hidden, device="cuda", dtype=td)
    s = torch.full((1,), 0.05, device="cuda")
    arn.norm(x, w, 1e-6, residual=res, fp8=fp8, scale=s)
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert arn.last_plan() == arn.norm_plan(dtype, rows, hidden, fused=fused, fp8=fp8,
                                            compute_units=cus)
