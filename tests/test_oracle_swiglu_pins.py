"""Pins of the oracle's SwiGLU (silu(gate) * up) against things other than
itself: torch's float64 SiLU (a library routine the oracle does not call),
the closed form sigmoid(ln k) = k / (k + 1), the odd-part identity
silu(g) - silu(-g) = g, limits, and hand-computed products that tell the
gate half from the up half."""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _bits(vals, dtype="bf16"):
    f = np.asarray(vals, np.float32)
    if dtype == "fp16":
        return f.astype(np.float16).view(np.uint16)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _vals(bits, dtype="bf16"):
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()


def test_silu_matches_torch_float64(orc):
    rng = np.random.default_rng(30)
    g = np.concatenate([rng.standard_normal(20000) * 4, rng.uniform(-60, 60, 2000),
                        [0.0, -0.0, 1e-300, -1e-300, 20.0, -20.0, 700.0, -700.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    got = np.array([orc.silu(float(v)) for v in g])
    assert np.allclose(got, ref, rtol=2e-15, atol=0)


def test_silu_far_negative_follows_g_exp_g(orc):
    """For g -> -inf, silu(g) = g / (1 + e^-g) = g e^g (1 - e^g + ...), so
    silu(g) / silu(g - 1) tends to e * g / (g - 1), and silu(g) keeps its
    magnitude e^g |g| down to fp64's subnormal range (about -745): no cliff
    where e^-g itself passes fp64's largest value (g below about -709.8)."""
    gs = [-600.0, -700.0, -709.0, -709.5, -710.0, -711.0, -720.0, -730.0]
    for g in gs:
        a, b = orc.silu(g), orc.silu(g - 1.0)
        assert a < 0.0 and b < 0.0
        # relative spacing of fp64 numbers near e^-740 is still below 1e-9
        assert a / b == pytest.approx(math.e * g / (g - 1.0), rel=1e-6)
    assert orc.silu(-800.0) == 0.0  # g e^g is below fp64's smallest subnormal


def test_silu_closed_forms(orc):
    for k in range(1, 12):
        g = math.log(k)
        assert orc.silu(g) == pytest.approx(g * k / (k + 1), rel=2e-15, abs=1e-300)
    assert orc.silu(0.0) == 0.0
    assert orc.silu(1e4) == 1e4           # sigmoid saturates at 1
    assert orc.silu(-1e4) == 0.0          # and at 0
    rng = np.random.default_rng(31)
    for g in rng.standard_normal(200) * 8:
        assert orc.silu(g) - orc.silu(-g) == pytest.approx(g, rel=1e-14, abs=1e-300)


def test_gate_times_up_hand_values(orc):
    """Row (gate | up) = (2, -1 | 3, 0.5): y = (3 * silu(2), 0.5 * silu(-1))
    with silu(2) = 2 / (1 + e^-2), silu(-1) = -1 / (1 + e)."""
    x = _bits([[2.0, -1.0, 3.0, 0.5]])
    r = orc.silu_and_mul("bf16", x)
    assert r["y"][0, 0] == pytest.approx(3 * 2 / (1 + math.exp(-2)), rel=1e-15)
    assert r["y"][0, 1] == pytest.approx(0.5 * -1 / (1 + math.e), rel=1e-15)


def test_up_of_one_gives_silu_and_padding_is_ignored(orc):
    rng = np.random.default_rng(32)
    d, stride = 100, 256
    x = np.full((4, stride), 0x7FA5, np.uint16)   # NaN padding after 2d
    g = _bits(rng.standard_normal((4, d)) * 3, "fp16")
    x[:, :d] = g
    x[:, d:2 * d] = _bits(np.ones((4, d)), "fp16")
    r = orc.silu_and_mul("fp16", x, d=d)
    expect = np.vectorize(orc.silu)(_vals(g, "fp16"))
    assert np.array_equal(r["y"], expect)
    assert np.all(np.isfinite(r["y"]))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_y16_is_rne_of_y(orc, dtype):
    rng = np.random.default_rng(33)
    x = _bits(rng.standard_normal((8, 64)) * 2, dtype)
    r = orc.silu_and_mul(dtype, x)
    if dtype == "fp16":
        ref = r["y"].astype(np.float16).view(np.uint16)
    else:
        ref = None
    if ref is not None:
        assert np.array_equal(r["y16"], ref)
    back = _vals(r["y16"], dtype)
    assert np.all(np.abs(back - r["y"]) <= np.abs(r["y"]) * 2.0**-8 + 1e-30)


def test_swiglu_fp8_dynamic_invariants(orc):
    rng = np.random.default_rng(34)
    x = _bits(rng.standard_normal((6, 2 * 300)) * 2)
    x[2] = 0
    r = orc.silu_and_mul("bf16", x, fp8_mode=O.FP8_DYNAMIC)
    for i in range(6):
        y = r["y"][i]
        amax = np.max(np.abs(y))
        if amax == 0:
            assert r["scales"][i] == 0 and np.all(r["q"][i] == 0)
            continue
        assert r["scales"][i] == np.float32(amax / 448)
        assert r["q"][i, int(np.argmax(np.abs(y)))] & 0x7F == 0x7E


def test_swiglu_fp8_static_exact_points(orc):
    """up = 1 and gate large (silu(g) = g exactly in fp64 for g >= 40) put
    y on chosen e4m3 grid points: codes exact."""
    grid = [64.0, 72.0, 80.0, 96.0, 112.0, 128.0, 160.0, 192.0, 224.0, 256.0, 320.0, 448.0]
    s = 0.5
    x = _bits([[v * s for v in grid] + [1.0] * len(grid)])
    r = orc.silu_and_mul("bf16", x, fp8_mode=O.FP8_STATIC, static_scale=s)
    for j, v in enumerate(grid):
        assert orc.e4m3_decode(int(r["q"][0, j])) == v


def test_split_halves_with_their_own_strides(orc):
    """Gate and up in separate arrays with different row strides give the
    same y as one [rows, 2d] tensor."""
    rng = np.random.default_rng(35)
    rows, d = 5, 48
    g = _bits(rng.standard_normal((rows, d)) * 2)
    u = _bits(rng.standard_normal((rows, d)) * 2)
    gate = np.full((rows, 64), 0x7FA5, np.uint16)
    up = np.full((rows, 96), 0x7FA5, np.uint16)
    gate[:, :d] = g
    up[:, :d] = u
    split = orc.silu_and_mul_split("bf16", gate, up, d=d)
    joined = orc.silu_and_mul("bf16", np.concatenate([g, u], axis=1))
    assert np.array_equal(split["y"], joined["y"])
