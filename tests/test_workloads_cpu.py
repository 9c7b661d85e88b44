"""Pins of the seeded input generator (workloads/): reproducibility, the
structure each workload states, and plausible moments.

The generator holds no operator arithmetic; both the oracle and the HIP
path are fed from it, and the stored static scales under tests/golden/ were
calibrated on its seed-0 draw, so the draw itself is pinned here."""
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from tests.golden.make_golden import digest

HERE = os.path.dirname(os.path.abspath(__file__))
DIGESTS = json.load(open(os.path.join(HERE, "golden", "workload_digests.json")))["workloads"]


def _vals(bits, dtype):
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16) \
        .double().numpy()


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_stored_digest_of_the_first_rows(name):
    """The first rows (up to 256) hash to the value tests/golden/make_golden.py
    stored: the same seed gives the same bytes on every run and machine."""
    w = W.WORKLOADS[name]
    rows = DIGESTS[name]["rows"]
    assert rows == min(256, w.rows)
    assert digest(W.make(w, rows=rows, seed=0)) == DIGESTS[name]["sha256"]


def test_regeneration_is_byte_identical_and_seeds_differ():
    w = W.WORKLOADS["fused_add_rmsnorm_bf16_65536x2880_stride4096"]
    a, b = W.make(w, rows=300), W.make(w, rows=300)
    for k in ("x", "residual", "weight"):
        assert np.array_equal(a[k], b[k]), k
    c = W.make(w, rows=300, seed=1)
    assert not np.array_equal(a["x"], c["x"])
    assert not np.array_equal(a["x"][:, :w.hidden], a["residual"][:, :w.hidden])


def test_any_row_range_regenerates_alone():
    """Rows are keyed by blocks of 256, so rows [300, 700) drawn alone equal
    the same rows of a longer draw (full-size parity samples rows this way)."""
    w = W.WORKLOADS["fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168"]
    whole = W.make(w, rows=700)
    part = W.make_rows(w, 300, 700)
    for k in ("x", "residual"):
        assert np.array_equal(part[k], whole[k][300:700]), k
    assert np.array_equal(part["weight"], whole["weight"])


def test_decode_row_counts_are_prefixes_of_the_256_row_draw():
    for name in ("fused_add_rmsnorm_fp8_static_fp16_decode_x16384",
                 "silu_and_mul_fp8_static_bf16_decode_x6656"):
        w = W.WORKLOADS[name]
        full = W.make(w, rows=256)
        assert w.row_counts == (1, 8, 64, 256)
        for r in w.row_counts:
            d = W.make(w, rows=r)
            for k, v in d.items():
                if v is not None and k != "weight":
                    assert np.array_equal(v, full[k][:r]), (name, r, k)


def test_outlier_columns_are_eight_fixed_distinct_columns():
    """C4: 8 distinct columns of x, the same in every row, carry x * 50;
    the residual and the other columns do not."""
    w = W.WORKLOADS["fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168"]
    cols = W.outlier_columns(w)
    assert cols.size == 8 == np.unique(cols).size
    assert np.all((cols >= 0) & (cols < w.hidden))
    assert np.array_equal(cols, W.outlier_columns(w))
    d = W.make(w, rows=512)
    x = _vals(d["x"], w.dtype)
    res = _vals(d["residual"], w.dtype)
    col_std = x.std(axis=0)
    assert np.all(col_std[cols] > 40) and np.all(col_std[cols] < 60)
    others = np.setdiff1d(np.arange(w.hidden), cols)
    assert np.all(col_std[others] < 1.4)
    # the 8 largest |x| of almost every row fall in the outlier columns
    top = np.argsort(-np.abs(x), axis=1)[:, :8]
    frac = np.mean([np.isin(cols, t).sum() >= 6 for t in top])
    assert frac > 0.95
    assert res.std(axis=0)[cols].max() < 1.4


def test_padding_holds_the_sentinel():
    for name in ("fused_add_rmsnorm_bf16_65536x3840_stride4096",
                 "fused_add_rmsnorm_bf16_65536x2880_stride4096"):
        w = W.WORKLOADS[name]
        d = W.make(w, rows=20)
        for k in ("x", "residual"):
            assert d[k].shape == (20, w.stride)
            assert np.all(d[k][:, w.hidden:] == W.PAD_SENTINEL)
            assert np.all(d[k][:, :w.hidden] != W.PAD_SENTINEL)


def _check_moments(v, mean, var, what):
    """Sample mean and variance within 5 standard errors (the 16-bit rounding
    of the draws moves them by far less)."""
    n = v.size
    m, s2 = float(v.mean()), float(v.var())
    fourth = float(np.mean((v - m) ** 4))
    assert abs(m - mean) <= 5 * math.sqrt(var / n), (what, m)
    assert abs(s2 - var) <= 5 * math.sqrt(max(fourth - var * var, 1e-30) / n), (what, s2)


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_moments(name):
    w = W.WORKLOADS[name]
    rows = min(64, w.rows)
    d = W.make(w, rows=rows)
    H = w.hidden
    if w.is_sum:
        for g, p in enumerate(d["parts"]):
            _check_moments(_vals(p[:, :H], w.dtype).ravel(), 0.0, w.x_std ** 2, f"part {g}")
    else:
        x = _vals(d["x"][:, :w.in_width], w.dtype)
        if w.outliers:
            x = np.delete(x, W.outlier_columns(w), axis=1)
        _check_moments(x.ravel(), 0.0, w.x_std ** 2, "x")
    if w.has_residual:
        _check_moments(_vals(d["residual"][:, :H], w.dtype).ravel(), 0.0, w.res_std ** 2,
                       "residual")
    if d["weight"] is not None:
        wv = _vals(d["weight"], w.dtype)
        mean, var = {"1+0.1n": (1.0, 0.01), "u(0.5,1.5)": (1.0, 1.0 / 12)}[w.weight]
        _check_moments(wv, mean, var, "weight")
        if w.weight == "u(0.5,1.5)":
            assert wv.min() >= 0.5 and wv.max() <= 1.5


def test_gemm_inputs_shapes_and_ranges():
    g = W.GEMMS["fp8_gemm_o_16384x2048"]
    d = W.make_gemm(g, 8)
    assert d["a"].shape == (8, g.k) and d["b"].shape == (g.n, g.k)
    assert not np.any((d["a"] & 0x7F) == 0x7F) and not np.any((d["b"] & 0x7F) == 0x7F)
    assert np.all((d["scale_a"] >= 0.01) & (d["scale_a"] <= 0.1))
    assert np.all((d["scale_b"] >= 0.001) & (d["scale_b"] <= 0.01))
    d2 = W.make_gemm(g, 8)
    assert all(np.array_equal(d[k], d2[k]) for k in d)
