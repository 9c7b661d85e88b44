"""The GEMM entry point that allocates nothing
(arn_fp8_gemm_preshuffled_noalloc, its split-K partials in the library's
own device array) against the workspace entry point
(arn_fp8_gemm_preshuffled_ws) on the same inputs: two calls in a row, the
second smaller, each equal bit for bit to the workspace call and within the
GEMM tolerance of the oracle; repeated calls; the size limit."""
import numpy as np
import pytest
import torch

from tests._helpers import bits, gemm_ref, gemm_tol, values16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _codes(rng, rows, cols, std):
    f = torch.from_numpy((rng.standard_normal((rows, cols)) * std).astype(np.float32))
    return f.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _data(m, n, k, seed):
    rng = np.random.default_rng(seed)
    a = _codes(rng, m, k, 24.0)
    b = _codes(rng, n, k, 6.0)
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    return a, sa, b, sb


def test_noalloc_matches_the_workspace_entry_point(orc):
    import residual_add_rmsnorm_amd as arn

    # the second call is smaller; both split K (plan checked)
    for m, n, k in ((64, 2304, 16384), (8, 1024, 2048)):
        print(f"\n[noalloc] m {m} n {n} k {k}", flush=True)
        a, sa, b, sb = _data(m, n, k, seed=m + n)
        ad, sad, sbd = (torch.from_numpy(v).cuda() for v in (a, sa, sb))
        bp = arn.fp8_weight_preshuffle(torch.from_numpy(b).cuda())
        ws = arn.fp8_gemm_workspace(m, n, k)
        want = arn.fp8_gemm(ad, sad, bp, sbd, workspace=ws)
        plan_ws = arn.last_plan()
        out = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = arn.fp8_gemm_preshuffled_noalloc(ad, sad, bp, sbd, out=out)
        plan = arn.last_plan()
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert plan == plan_ws and "/splits1/" not in plan, (plan, plan_ws)
        assert torch.equal(got, want)
        ref = gemm_ref(orc, a, sa, b, sb)
        err = np.abs(values16(bits(got), "bf16") - ref["c"])
        assert np.all(err <= gemm_tol(ref, k))


def test_noalloc_repeats_and_refuses_oversized_shapes():
    import residual_add_rmsnorm_amd as arn

    m, n, k = 16, 2304, 4096
    a, sa, b, sb = _data(m, n, k, seed=5)
    ad, sad, sbd = (torch.from_numpy(v).cuda() for v in (a, sa, sb))
    bp = arn.fp8_weight_preshuffle(torch.from_numpy(b).cuda())
    first = arn.fp8_gemm_preshuffled_noalloc(ad, sad, bp, sbd).clone()
    for _ in range(5):
        assert torch.equal(arn.fp8_gemm_preshuffled_noalloc(ad, sad, bp, sbd), first)
    # past the array (m = 64 serves n up to 4032): refused, nothing launched
    big = arn.fp8_weight_preshuffle(torch.zeros(4096, k, dtype=torch.uint8, device="cuda"))
    a64 = torch.zeros(64, k, dtype=torch.uint8, device="cuda")
    s1 = torch.ones(1, device="cuda")
    with pytest.raises(arn.ArnError) as e:
        arn.fp8_gemm_preshuffled_noalloc(a64, s1, big, s1)
    assert e.value.status == 2
    # the array was left ready: the earlier shape still gives the same bits
    assert torch.equal(arn.fp8_gemm_preshuffled_noalloc(ad, sad, bp, sbd), first)
