"""The binding's row views (the native row_view behind every entry point)
against brute force over element offsets, and its refusals without a GPU.

A view is served when its elements, taken in index order as rows of
`hidden`, sit at offset r * pitch + j from the first element for one pitch
(the layouts of flatten_to_2d_is_free on the vLLM API page
"vllm.kernels.aiter_ops", plus a padded pitch); anything else must be
refused, since the binding never copies.
"""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import residual_add_rmsnorm_amd as arn


def _brute(t):
    """(rows, hidden, pitch) from the element offsets alone, or None when no
    single pitch with unit column steps describes the view."""
    hidden = t.shape[-1]
    rows = int(np.prod(t.shape[:-1], dtype=np.int64))
    idx = np.indices(t.shape).reshape(t.dim(), -1)
    off = (np.asarray(t.stride(), dtype=np.int64)[:, None] * idx).sum(0).reshape(rows, hidden)
    if hidden > 1 and not (np.diff(off, axis=1) == 1).all():
        return None
    if rows == 1:
        return rows, hidden, hidden
    steps = np.diff(off[:, 0])
    if not (steps == steps[0]).all():
        return None
    pitch = int(steps[0])
    if pitch < hidden:
        return None
    return rows, hidden, pitch


@st.composite
def views(draw):
    nd = draw(st.integers(1, 4))
    shape = [draw(st.integers(1, 5)) for _ in range(nd)]
    t = torch.empty(shape, dtype=torch.bfloat16)
    for _ in range(draw(st.integers(0, 3))):
        op = draw(st.sampled_from(["transpose", "slice", "narrow_last", "expand", "unsqueeze"]))
        d = t.dim()
        if op == "transpose" and d >= 2:
            a, b = draw(st.integers(0, d - 1)), draw(st.integers(0, d - 1))
            t = t.transpose(a, b)
        elif op == "slice":
            a = draw(st.integers(0, d - 1))
            step = draw(st.integers(1, 3))
            t = t[(slice(None),) * a + (slice(None, None, step),)]
        elif op == "narrow_last" and t.shape[-1] > 1:
            n = draw(st.integers(1, t.shape[-1]))
            t = t.narrow(-1, draw(st.integers(0, t.shape[-1] - n)), n)
        elif op == "expand":
            ones = [i for i in range(d) if t.shape[i] == 1]
            if ones:
                i = draw(st.sampled_from(ones))
                size = list(t.shape)
                size[i] = draw(st.integers(2, 3))
                t = t.expand(size)
        elif op == "unsqueeze" and d < 5:
            t = t.unsqueeze(draw(st.integers(0, d)))
    return t


@settings(max_examples=600, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(views())
def test_row_view_matches_brute_force(t):
    want = _brute(t)
    if want is None:
        with pytest.raises(ValueError):
            arn._rows(t, "x")
    else:
        assert arn._rows(t, "x") == want, (tuple(t.shape), t.stride())


def test_row_view_cases():
    assert arn._rows(torch.empty(4, 6, 100, dtype=torch.bfloat16), "x") == (24, 100, 100)
    padded = torch.empty(16, 128, dtype=torch.float16)[:, :96]
    assert arn._rows(padded, "x") == (16, 96, 128)
    assert arn._rows(torch.empty(96, dtype=torch.bfloat16), "x") == (1, 96, 96)
    assert arn._rows(torch.empty(0, 64, dtype=torch.bfloat16), "x")[:2] == (0, 64)
    with pytest.raises(ValueError, match="at least one dimension"):
        arn._rows(torch.empty((), dtype=torch.bfloat16), "x")
    with pytest.raises(ValueError, match="unit stride"):
        arn._rows(torch.empty(8, 96, dtype=torch.bfloat16).t(), "x")
    with pytest.raises(ValueError, match="without a copy"):
        arn._rows(torch.empty(4, 8, 96, dtype=torch.bfloat16).transpose(0, 1), "x")
    with pytest.raises(ValueError, match="rows overlap"):
        arn._rows(torch.empty(1, 96, dtype=torch.bfloat16).expand(4, 96), "x")


def test_every_native_entry_point_refuses_host_tensors():
    x = torch.zeros(2, 8, dtype=torch.bfloat16)
    w = torch.ones(8, dtype=torch.bfloat16)
    s = torch.ones(1)
    codes = torch.zeros(2, 8, dtype=torch.uint8)
    calls = [
        lambda: arn.rmsnorm(x, w, 1e-6),
        lambda: arn.fused_add_rmsnorm(x, x.clone(), w, 1e-6),
        lambda: arn.rmsnorm_fp8(x, w, 1e-6, scale=s),
        lambda: arn.fused_add_rmsnorm_fp8(x, x.clone(), w, 1e-6, dynamic=True),
        lambda: arn.norm(x, w, 1e-6, variance_size=4),
        lambda: arn.silu_and_mul(x),
        lambda: arn.silu_and_mul_fp8(x, dynamic=True),
        lambda: arn.fp8_gemm(codes, s, codes, s),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU device"):
            call()
