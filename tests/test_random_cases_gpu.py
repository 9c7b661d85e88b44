"""Property-style parity over randomly drawn shapes and modes (hypothesis,
derandomized so the case list is fixed), and the library driven from
several host threads at once.

Each drawn case goes through the same checks as the hand-picked parity
tests (tests/test_parity_gpu.py::run_case, tests/test_gemm_gpu.py::check)."""
import threading

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads as W
from tests._helpers import dev

pytestmark = pytest.mark.gpu

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                    suppress_health_check=list(HealthCheck))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


hidden_st = st.one_of(st.integers(1, 9000), st.integers(1, 1100).map(lambda v: 8 * v))


@SETTINGS
@given(dtype=st.sampled_from(["bf16", "fp16"]), rows=st.integers(1, 300), hidden=hidden_st,
       pad=st.integers(0, 17), fp8=st.sampled_from([None, "static", "dynamic"]),
       fused=st.booleans(), weighted=st.booleans(), eps=st.sampled_from([1e-6, 1e-5, 0.1]),
       seed=st.integers(0, 2**31 - 1))
def test_random_norm_cases(orc, dtype, rows, hidden, pad, fp8, fused, weighted, eps, seed):
    from tests.test_parity_gpu import _random, run_case

    print(f"[case] norm {dtype} rows={rows} hidden={hidden} pad={pad} fp8={fp8} "
          f"fused={fused} weighted={weighted} eps={eps} seed={seed}", flush=True)
    stride = hidden + pad
    x = _random(dtype, rows, hidden, stride, seed)
    r = _random(dtype, rows, hidden, stride, seed + 1, std=2.0) if fused else None
    w = _random(dtype, 1, hidden, hidden, seed + 2)[0] if weighted else None
    run_case(orc, dtype=dtype, x=x, res=r, w=w, eps=eps, hidden=hidden, fp8=fp8,
             s=0.02 if fp8 == "static" else None)


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(rows=st.integers(1, 40), hidden=hidden_st, log2_scale=st.integers(-133, 120),
       fp8=st.sampled_from([None, "static", "dynamic"]), fused=st.booleans(),
       eps=st.sampled_from([0.0, 1e-38, 1e-30, 1e-6]), seed=st.integers(0, 2**31 - 1))
def test_random_bf16_magnitudes(orc, rows, hidden, log2_scale, fp8, fused, eps, seed):
    """bf16 rows of every magnitude bf16 holds (N(0,1) scaled by 2^-133 ..
    2^120, clipped to +-2^126), so the sum of squares may underflow or
    overflow fp32, with eps from 0 up: the same checks as every other case."""
    from tests.test_parity_gpu import run_case

    print(f"[case] magnitude bf16 rows={rows} hidden={hidden} 2^{log2_scale} fp8={fp8} "
          f"fused={fused} eps={eps} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)
    scale = 2.0 ** log2_scale

    def draw(mult):
        f = np.clip(rng.standard_normal((rows, hidden)) * scale * mult, -2.0**126, 2.0**126)
        return W.to_bits(f.astype(np.float32), "bf16")
    x = draw(1.0)
    r = draw(0.5) if fused else None
    w = W.to_bits(rng.uniform(0.5, 1.5, hidden).astype(np.float32), "bf16")
    run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=eps, hidden=hidden, fp8=fp8,
             s=2.0**-6 if fp8 == "static" else None)


@settings(max_examples=50, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(rows=st.integers(1, 16), hidden=st.integers(1, 520).map(lambda v: 8 * v),
       log2_x=st.integers(-133, 120), log2_w=st.integers(-133, 110),
       fp8=st.sampled_from(["static", "dynamic"]), fused=st.booleans(),
       eps=st.sampled_from([0.0, 1e-38, 1e-6]), log2_s=st.integers(-126, 127),
       seed=st.integers(0, 2**31 - 1))
def test_random_bf16_weight_magnitudes(orc, rows, hidden, log2_x, log2_w, fp8, fused, eps,
                                       log2_s, seed):
    """e4m3 outputs of bf16 rows whose activations and weights both range
    over every magnitude bf16 holds, so the products r * w and the dynamic
    scale may leave fp32's range in either direction; static scales over
    the normal fp32 range.  Weights stay below 2^111 so that |y| stays below
    2^128, which the static kind forms in fp32."""
    from tests.test_parity_gpu import run_case

    print(f"[case] weight magnitude bf16 rows={rows} hidden={hidden} x 2^{log2_x} w 2^{log2_w} "
          f"fp8={fp8} fused={fused} eps={eps} s 2^{log2_s} seed={seed}", flush=True)
    rng = np.random.default_rng(seed)

    def draw(shape, log2_scale, mult=1.0):
        f = np.clip(rng.standard_normal(shape) * 2.0**log2_scale * mult, -2.0**126, 2.0**126)
        return W.to_bits(f.astype(np.float32), "bf16")
    x = draw((rows, hidden), log2_x)
    r = draw((rows, hidden), log2_x, 0.5) if fused else None
    w = draw((hidden,), log2_w)
    run_case(orc, dtype="bf16", x=x, res=r, w=w, eps=eps, hidden=hidden, fp8=fp8,
             s=2.0**log2_s if fp8 == "static" else None)


@SETTINGS
@given(m=st.integers(1, 64), n=st.integers(1, 3000), k16=st.integers(1, 512),
       layout=st.sampled_from(["rowmajor", "preshuffled", "splitk"]),
       out=st.sampled_from(["bf16", "fp16"]), seed=st.integers(0, 2**31 - 1))
def test_random_gemm_cases(orc, m, n, k16, layout, out, seed):
    import residual_add_rmsnorm_amd as arn
    from tests.test_gemm_gpu import check

    k = 16 * k16
    print(f"[case] gemm m={m} n={n} k={k} layout={layout} out={out} seed={seed}", flush=True)
    ws = arn.fp8_gemm_workspace(m, n, k) if layout == "splitk" else None
    check(orc, m, n, k, out=out, seed=seed % 100000, pre=layout != "rowmajor", workspace=ws)


def test_threads_each_on_their_own_stream():
    """Four host threads, each with its own stream and buffers, call the
    norm and the split-K GEMM 25 times; every result equals the same call
    made alone (the kernels are deterministic, so bit for bit)."""
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(90)
    jobs = []
    for t in range(4):
        x = dev(W.to_bits(rng.standard_normal((64, 4096)).astype(np.float32), "bf16"), "bf16")
        r = dev(W.to_bits(rng.standard_normal((64, 4096)).astype(np.float32), "bf16"), "bf16")
        w = dev(W.to_bits((1 + 0.1 * rng.standard_normal(4096)).astype(np.float32), "bf16"),
                "bf16")
        a = torch.from_numpy(W.e4m3_codes(rng.standard_normal((16, 2048)) * 8)).cuda()
        b = arn.fp8_weight_preshuffle(torch.from_numpy(
            W.e4m3_codes(rng.standard_normal((2304, 2048)) * 4)).cuda())
        sa = torch.full((16,), 0.05, device="cuda")
        sb = torch.full((2304,), 0.004, device="cuda")
        jobs.append((x, r, w, a, sa, b, sb, arn.fp8_gemm_workspace(16, 2304, 2048)))

    def one(job, stream):
        x, r, w, a, sa, b, sb, ws = job
        with torch.cuda.stream(stream):
            rr = r.clone()
            y = arn.fused_add_rmsnorm(x, rr, w, 1e-6)
            c = arn.fp8_gemm(a, sa, b, sb, workspace=ws)
        stream.synchronize()
        return rr, y, c

    streams = [torch.cuda.Stream() for _ in jobs]
    ref = [one(j, s) for j, s in zip(jobs, streams)]
    errors = []

    def worker(i):
        try:
            for _ in range(25):
                got = one(jobs[i], streams[i])
                for g, e in zip(got, ref[i]):
                    if not torch.equal(g, e):
                        errors.append(i)
                        return
        except Exception as ex:  # surfaced below
            errors.append(repr(ex))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
