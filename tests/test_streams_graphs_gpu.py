"""The library on non-default streams and inside HIP graphs.

Each call enqueues one kernel on torch's current stream, so it must work on
any stream and be capturable.  A captured fused call updates the residual in
place, so replay k must equal k applications of the operator; every replay is
checked against the oracle iterated on the CPU, with eager work and
synchronisations between replays.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests._helpers import assert_codes_close, assert_y_close, bits, codes, dev, gemm_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _inputs(rows=96, hidden=4096, seed=40):
    rng = np.random.default_rng(seed)
    x = W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16")
    r = W.to_bits(rng.standard_normal((rows, hidden)).astype(np.float32), "bf16")
    w = W.to_bits((1 + 0.1 * rng.standard_normal(hidden)).astype(np.float32), "bf16")
    return x, r, w


def test_non_default_stream(orc):
    import residual_add_rmsnorm_amd as arn

    x, r, w = _inputs()
    s = torch.cuda.Stream()
    xd, rd, wd = dev(x, "bf16"), dev(r, "bf16"), dev(w, "bf16")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y = arn.fused_add_rmsnorm(xd, rd, wd, 1e-6)
    s.synchronize()
    ref = orc.add_rmsnorm("bf16", x, r, w, 1e-6)
    assert np.array_equal(bits(rd), ref["r16"])
    assert_y_close(bits(y), ref["y"], "bf16")


def test_graph_replays_match_iterated_oracle(orc):
    import residual_add_rmsnorm_amd as arn

    x, r, w = _inputs()
    xd, rd, wd = dev(x, "bf16"), dev(r, "bf16"), dev(w, "bf16")
    out = torch.empty_like(xd)
    q = torch.empty(xd.shape, dtype=torch.float8_e4m3fn, device="cuda")
    sc = torch.empty(xd.shape[0], dtype=torch.float32, device="cuda")
    rd2 = rd.clone()
    # warm up on a side stream, as graph capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tmp = rd.clone()
        arn.fused_add_rmsnorm(xd, tmp, wd, 1e-6, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        arn.fused_add_rmsnorm(xd, rd, wd, 1e-6, out=out)
        arn.fused_add_rmsnorm_fp8(xd, rd2, wd, 1e-6, dynamic=True, out=q, scales_out=sc)

    res_ref, res_ref2 = r.copy(), r.copy()
    for k in range(4):
        g.replay()
        torch.cuda.synchronize()
        ref = orc.add_rmsnorm("bf16", x, res_ref, w, 1e-6)
        ref2 = orc.add_rmsnorm("bf16", x, res_ref2, w, 1e-6, fp8_mode=O.FP8_DYNAMIC)
        res_ref, res_ref2 = ref["r16"], ref2["r16"]
        assert np.array_equal(bits(rd), res_ref), f"replay {k}: residual"
        assert_y_close(bits(out), ref["y"], "bf16", what=f"replay {k}: y")
        assert np.array_equal(bits(rd2), res_ref2), f"replay {k}: fp8 residual"
        assert_codes_close(codes(q), ref2["q"], what=f"replay {k}: codes")
        # eager work between replays
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        del junk


def _gemm_inputs(m, n, k, seed):
    rng = np.random.default_rng(seed)
    f = lambda rows, std: W.e4m3_codes(rng.standard_normal((rows, k)) * std)
    a, b = f(m, 24.0), f(n, 6.0)
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    return a, b, sa, sb


def _gemm_tol(ref, k):
    from tests._helpers import gemm_tol

    return gemm_tol(ref, k)


@pytest.mark.parametrize("split", [False, True])
def test_gemm_non_default_stream(orc, split):
    import residual_add_rmsnorm_amd as arn
    from tests._helpers import values16

    m, n, k = 16, 2304, 4096
    a, b, sa, sb = _gemm_inputs(m, n, k, 41)
    ad, sad, sbd = (torch.from_numpy(v).cuda() for v in (a, sa, sb))
    bw = arn.fp8_weight_preshuffle(torch.from_numpy(b).cuda())
    ws = arn.fp8_gemm_workspace(m, n, k) if split else None
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = arn.fp8_gemm(ad, sad, bw, sbd, workspace=ws)
    s.synchronize()
    assert ("splits1" not in arn.last_plan()) == split
    ref = gemm_ref(orc, a, sa, b, sb)
    assert np.all(np.abs(values16(bits(c), "bf16") - ref["c"]) <= _gemm_tol(ref, k))


def test_decode_graph_with_split_gemm(orc):
    """A captured decode step -- fused add + norm to dynamic e4m3, then the
    split-K GEMM on those codes -- replayed several times with eager work and
    synchronisations in between: every replay equals the eager result (the
    split counters must come back to zero after each replay)."""
    import residual_add_rmsnorm_amd as arn

    x, r, w = _inputs(rows=16, hidden=2048, seed=42)
    _, b, _, sb = _gemm_inputs(1, 2304, 2048, 43)
    xd, wd = dev(x, "bf16"), dev(w, "bf16")
    rd = dev(r, "bf16")
    bw = arn.fp8_weight_preshuffle(torch.from_numpy(b).cuda())
    sbd = torch.from_numpy(sb).cuda()
    ws = arn.fp8_gemm_workspace(16, 2304, 2048)
    q = torch.empty(xd.shape, dtype=torch.float8_e4m3fn, device="cuda")
    sc = torch.empty(16, dtype=torch.float32, device="cuda")
    c = torch.empty((16, 2304), dtype=torch.bfloat16, device="cuda")

    def step():
        arn.fused_add_rmsnorm_fp8(xd, rd, wd, 1e-6, dynamic=True, out=q, scales_out=sc)
        arn.fp8_gemm(q, sc, bw, sbd, out=c, workspace=ws)

    # eager reference for k applications
    r0 = rd.clone()
    eager = []
    for _ in range(4):
        step()
        eager.append((rd.clone(), c.clone()))
    torch.cuda.synchronize()
    assert "splits1" not in arn.last_plan()
    rd.copy_(r0)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tmp_r = rd.clone()
        arn.fused_add_rmsnorm_fp8(xd, tmp_r, wd, 1e-6, dynamic=True, out=q, scales_out=sc)
        arn.fp8_gemm(q, sc, bw, sbd, out=c, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    rd.copy_(r0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        g.replay()
        junk = torch.randn(1024, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(rd, eager[i][0]), f"replay {i}: residual"
        assert torch.equal(c, eager[i][1]), f"replay {i}: GEMM output"
        del junk
