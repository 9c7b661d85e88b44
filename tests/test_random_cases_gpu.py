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


@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@settings(max_examples=25, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(rows=st.integers(1, 12),
       hidden=st.one_of(st.integers(1, 3000), st.integers(1, 520).map(lambda v: 8 * v)),
       kfrac=st.floats(0.0, 1.0), fused=st.booleans(), eps=st.sampled_from([0.0, 1e-38, 1e-6]),
       seed=st.integers(0, 2**31 - 1))
def test_random_variance_size_magnitudes(orc, dtype, fp8, rows, hidden, kfrac, fused, eps,
                                         seed):
    """The variance-size override with the channels inside the mean and the
    ones outside it at independent magnitudes, each a power of two drawn from
    the seed over bf16's whole range (fp16 rows: over fp16's), every output
    kind, with and without the residual.  The stored
    residual is compared on every row; y, codes and scales on the rows whose
    y is finite (and, for 16-bit outputs and bf16 static e4m3, below 2^127,
    where y itself is formed in fp32 and the dtype's largest value is
    near)."""
    import residual_add_rmsnorm_amd as arn
    from tests._helpers import (assert_codes_close, assert_scales_close, assert_y_close,
                                bits, codes)
    import oracle as O

    k = 1 + int(kfrac * (hidden - 1))
    rng = np.random.default_rng(seed)
    if dtype == "fp16":
        top = 15
        log2_in = int(rng.integers(-24, top + 1))
        lo = int(rng.integers(-24, top + 1))
    else:
        top = 126
        # mean-square channels tiny, ordinary or huge with equal odds (the
        # first and last need the rescaled sum unless eps dominates)
        band = [(-133, -49), (-48, 59), (60, 126)][int(rng.integers(0, 3))]
        log2_in = int(rng.integers(band[0], band[1] + 1))
        lo = int(rng.integers(-133, top + 1))
    log2_s = int(rng.integers(-126, 128))
    s = 2.0**log2_s
    print(f"[case] variance size {dtype} rows={rows} hidden={hidden} k={k} in 2^{log2_in} "
          f"out 2^{lo} fp8={fp8} fused={fused} eps={eps} s 2^{log2_s} seed={seed}", flush=True)
    lim = 1.9 * 2.0**top

    def draw(mult):
        f = rng.standard_normal((rows, hidden)) * mult
        f[:, :k] *= 2.0**log2_in
        f[:, k:] *= 2.0**lo
        return W.to_bits(np.clip(f, -lim, lim).astype(np.float32), dtype)
    x = draw(1.0)
    r = draw(0.5) if fused else None
    w = W.to_bits(rng.uniform(0.5, 1.5, hidden).astype(np.float32), dtype)
    xd, wd = dev(x, dtype), dev(w, dtype)
    rd = dev(r, dtype) if fused else None
    kw = dict(fp8="dynamic") if fp8 == "dynamic" else (
        dict(fp8="static", scale=torch.tensor([s], device="cuda")) if fp8 else {})
    out = arn.norm(xd, wd, eps, residual=rd, variance_size=k, **kw)
    torch.cuda.synchronize()
    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.add_rmsnorm(dtype, x, r, w, eps, fp8_mode=mode, static_scale=s,
                          variance_size=k)
    if fused:
        assert np.array_equal(bits(rd), ref["r16"]), "stored residual not bit-exact"
    ay = np.abs(ref["y"])
    ok = np.all(np.isfinite(ay), axis=1)
    if fp8 is None:
        ok &= np.all(ay < (2.0**127 if dtype == "bf16" else 65504.0), axis=1)
    elif fp8 == "static" and dtype == "bf16":
        ok &= np.all(ay < 2.0**127, axis=1)
    if fp8 == "dynamic":
        q, sc = out
        assert_scales_close(sc.cpu().numpy()[ok], ref["scales"][ok], dtype)
        assert_codes_close(codes(q)[ok], ref["q"][ok])
    elif fp8 == "static":
        assert_codes_close(codes(out[0])[ok], ref["q"][ok])
    else:
        assert_y_close(bits(out)[ok], ref["y"][ok], dtype)


@pytest.mark.parametrize("fp8", [None, "static", "dynamic"])
@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(rows=st.integers(1, 10),
       d=st.one_of(st.integers(1, 3000), st.integers(1, 520).map(lambda v: 8 * v)),
       seed=st.integers(0, 2**31 - 1))
def test_random_glu_magnitudes(orc, fp8, rows, d, seed):
    """bf16 SwiGLU rows whose gates and up values are each a power of two
    drawn from the seed over bf16's whole range (a third of the gates
    drawn below -80, where exp(-|g|) nears fp32's subnormal range), times
    N(0, 1), with random signs; static scales over the normal fp32 range.
    Rows with an output at or above 2^127 are left out for the 16-bit and
    static kinds, which form y in fp32, and dynamic rows whose scale rounds
    to zero while an output is exactly zero (its code is e4m3(0 / 0))."""
    import residual_add_rmsnorm_amd as arn
    from tests._helpers import assert_codes_close, assert_scales_close, assert_y_close, bits, codes
    import oracle as O

    rng = np.random.default_rng(seed)
    log2_s = int(rng.integers(-126, 128))
    s = 2.0**log2_s
    gate = np.empty((rows, d))
    up = np.empty((rows, d))
    for i in range(rows):
        lg, lu = int(rng.integers(-133, 127)), int(rng.integers(-133, 127))
        gate[i] = rng.standard_normal(d) * 2.0**lg
        if rng.random() < 1 / 3:
            gate[i] = -rng.uniform(80, 2.0**int(rng.integers(7, 20)), d)
        up[i] = rng.standard_normal(d) * 2.0**lu
    lim = 1.9 * 2.0**126
    x = W.to_bits(np.clip(np.concatenate([gate, up], axis=1), -lim, lim).astype(np.float32),
                  "bf16")
    print(f"[case] glu magnitudes rows={rows} d={d} fp8={fp8} s 2^{log2_s} seed={seed}",
          flush=True)
    xd = dev(x, "bf16")
    if fp8 == "dynamic":
        out = arn.silu_and_mul_fp8(xd, dynamic=True)
    elif fp8 == "static":
        out = arn.silu_and_mul_fp8(xd, scale=torch.tensor([s], device="cuda"))
    else:
        out = arn.silu_and_mul(xd)
    torch.cuda.synchronize()
    mode = {None: O.FP8_NONE, "static": O.FP8_STATIC, "dynamic": O.FP8_DYNAMIC}[fp8]
    ref = orc.silu_and_mul("bf16", x, d=d, fp8_mode=mode, static_scale=s)
    ok = np.all(np.isfinite(ref["y"]), axis=1)
    if fp8 != "dynamic":
        ok &= np.all(np.abs(ref["y"]) < 2.0**127, axis=1)
    else:
        # a scale that rounds to zero under an exact-zero output: 0 / 0
        ok &= ~((ref["scales"] == 0) & np.any(ref["y"] == 0, axis=1) & np.any(ref["y"] != 0, axis=1))
    if fp8 == "dynamic":
        q, sc = out
        assert_scales_close(sc.cpu().numpy()[ok], ref["scales"][ok], "bf16")
        assert_codes_close(codes(q)[ok], ref["q"][ok])
    elif fp8 == "static":
        q = out[0] if isinstance(out, tuple) else out
        assert_codes_close(codes(q)[ok], ref["q"][ok])
    else:
        assert_y_close(bits(out)[ok], ref["y"][ok], "bf16")


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
