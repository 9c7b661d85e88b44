"""The tuning aids of include/arn_tuning.h hold per-thread settings: a
shape forced on one host thread never reaches another thread's calls."""
import threading

import numpy as np
import pytest
import torch

import workloads as W
from tests._helpers import assert_y_close, bits, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _run_in_threads(first, second):
    """first() sets its shape, then second() runs in another thread while
    that setting is in force, then first() continues."""
    forced, checked = threading.Event(), threading.Event()
    out, errors = {}, []

    def a():
        try:
            out["a"] = first(forced, checked)
        except BaseException as e:  # noqa: BLE001
            errors.append(e)
            forced.set()

    def b():
        try:
            assert forced.wait(60)
            out["b"] = second()
        except BaseException as e:  # noqa: BLE001
            errors.append(e)
        finally:
            checked.set()

    ts = [threading.Thread(target=a), threading.Thread(target=b)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(120)
    assert not any(t.is_alive() for t in ts), "a thread did not finish"
    if errors:
        raise errors[0]
    return out


def test_forced_tile_stays_on_its_thread(orc):
    import residual_add_rmsnorm_amd as arn

    w = W.WORKLOADS["rmsnorm_bf16_64x4096"]
    d = W.make(w)
    x, wt = dev(d["x"], w.dtype), dev(d["weight"], w.dtype)
    ref = orc.add_rmsnorm(w.dtype, d["x"], None, d["weight"], w.eps)
    arn.rmsnorm(x, wt, w.eps)
    auto = arn.last_plan()
    assert "/wpr1/nv16/" not in auto

    def first(forced, checked):
        arn.set_tile(1, 16)
        try:
            forced.set()
            assert checked.wait(60)
            y = arn.rmsnorm(x, wt, w.eps)
            torch.cuda.synchronize()
            return bits(y), arn.last_plan()
        finally:
            arn.set_tile(0, 0)

    def second():
        assert arn.last_plan() == ""         # a new thread has launched nothing yet
        y = arn.rmsnorm(x, wt, w.eps)
        torch.cuda.synchronize()
        return bits(y), arn.last_plan()

    out = _run_in_threads(first, second)
    assert "/wpr1/nv16/" in out["a"][1], out["a"][1]
    assert out["b"][1] == auto, out["b"][1]
    for y, _ in out.values():
        assert_y_close(y, ref["y"], w.dtype)
    arn.rmsnorm(x, wt, w.eps)
    assert arn.last_plan() == auto


def test_forced_gemm_shape_and_splits_stay_on_their_thread():
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(3)
    m, n, k = 16, 2304, 4096
    a = torch.from_numpy(rng.integers(0, 0x70, (m, k)).astype(np.uint8)).cuda()
    b = torch.from_numpy(rng.integers(0, 0x70, (n, k)).astype(np.uint8)).cuda()
    sa = torch.full((m,), 0.01, device="cuda")
    sb = torch.full((n,), 0.02, device="cuda")
    ws = arn.fp8_gemm_workspace(m, n, k)
    ref = arn.fp8_gemm(a, sa, b, sb, workspace=ws).clone()
    auto = arn.last_plan()
    assert "/nt4/waves16/" not in auto

    def first(forced, checked):
        arn.set_gemm_config(4, 16)
        arn.set_gemm_splits(1)
        try:
            forced.set()
            assert checked.wait(60)
            c = arn.fp8_gemm(a, sa, b, sb, workspace=ws)
            torch.cuda.synchronize()
            return c.clone(), arn.last_plan()
        finally:
            arn.set_gemm_config(0, 0)
            arn.set_gemm_splits(0)

    def second():
        c = arn.fp8_gemm(a, sa, b, sb, workspace=ws)
        torch.cuda.synchronize()
        return c.clone(), arn.last_plan()

    out = _run_in_threads(first, second)
    assert "/nt4/waves16/splits1/" in out["a"][1], out["a"][1]
    assert out["b"][1] == auto, out["b"][1]
    assert torch.equal(out["b"][0], ref)     # same shape, same bits
    assert torch.allclose(out["a"][0].float(), ref.float(), rtol=2**-6, atol=1e-2)
