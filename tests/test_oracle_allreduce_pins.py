"""Pins of the oracle's all-reduce reduction step (orc_sum_parts16): the
nparts partial rows are accumulated in fp32 in rank order and rounded once
to the 16-bit type, the reading taken for the reduction that a fused
all-reduce + residual add + RMSNorm kernel performs before the norm.

Checked against numpy's own fp32 arithmetic, against cases where the rank
order decides the result, and against the single-part identity."""
import numpy as np
import pytest
import torch

import oracle as O

BF16_TWO24, BF16_ONE, BF16_MTWO24 = 0x4B80, 0x3F80, 0xCB80   # 2^24, 1, -2^24
FP16_MAX, FP16_TINY, FP16_MMAX = 0x7BFF, 0x0001, 0xFBFF       # 65504, 2^-24, -65504


def _round16(f32, dtype):
    """fp32 -> 16-bit patterns, nearest even (numpy for fp16, torch for bf16)."""
    if dtype == "fp16":
        return f32.astype(np.float16).view(np.uint16)
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _decode32(bits, dtype):
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _is_nan16(bits, dtype):
    if dtype == "fp16":
        return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x03FF) != 0)
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x007F) != 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_one_part_is_identity(orc, dtype):
    """With one rank the reduction returns its input, for every pattern."""
    allv = np.arange(65536, dtype=np.uint16).reshape(256, 256)
    got = orc.sum_parts(dtype, [allv])
    nan = _is_nan16(allv, dtype)
    assert np.array_equal(_is_nan16(got, dtype), nan)
    assert np.array_equal(got[~nan], allv[~nan])


def test_rank_order_decides_bf16(orc):
    """2^24 + 1 rounds back to 2^24 in fp32: in rank order (2^24, 1, -2^24)
    the total is 0; with the ranks permuted to (2^24, -2^24, 1) it is 1."""
    p = [np.array([[v]], np.uint16) for v in (BF16_TWO24, BF16_ONE, BF16_MTWO24)]
    assert orc.sum_parts("bf16", p)[0, 0] == 0x0000
    assert orc.sum_parts("bf16", [p[0], p[2], p[1]])[0, 0] == BF16_ONE
    assert orc.sum_parts("bf16", p[::-1])[0, 0] == BF16_ONE


def test_rank_order_decides_fp16(orc):
    """65504 + 2^-24 rounds back to 65504 in fp32."""
    p = [np.array([[v]], np.uint16) for v in (FP16_MAX, FP16_TINY, FP16_MMAX)]
    assert orc.sum_parts("fp16", p)[0, 0] == 0x0000
    assert orc.sum_parts("fp16", [p[0], p[2], p[1]])[0, 0] == FP16_TINY


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("nparts", [2, 3, 8])
def test_random_parts_match_numpy_fp32(orc, dtype, nparts):
    """Random partial rows (wide exponent spread, row padding) against
    numpy's sequential float32 additions and nearest-even rounding."""
    rng = np.random.default_rng(nparts * 7 + (dtype == "fp16"))
    rows, hidden, stride = 33, 300, 320
    parts = []
    for g in range(nparts):
        v = (rng.standard_normal((rows, stride)) * np.exp2(rng.integers(-12, 12, (rows, stride))))
        if dtype == "fp16":
            b = v.astype(np.float16).view(np.uint16)
        else:
            b = _round16(v.astype(np.float32), "bf16")
        b[:, hidden:] = 0x7FC1          # padding (NaN) must not be read
        parts.append(b)
    got = orc.sum_parts(dtype, parts, hidden=hidden)
    with np.errstate(over="ignore", invalid="ignore"):
        acc = _decode32(parts[0][:, :hidden], dtype)
        for b in parts[1:]:
            acc = (acc + _decode32(b[:, :hidden], dtype)).astype(np.float32)
        ref = _round16(acc, dtype)
    nan = np.isnan(acc)
    assert np.array_equal(_is_nan16(got, dtype), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_composition_is_add_rmsnorm_of_the_sum(orc):
    """sum_add_rmsnorm = add_rmsnorm applied to the reduced rows; with one
    part it is add_rmsnorm of that part."""
    rng = np.random.default_rng(5)
    x = _round16(rng.standard_normal((9, 128)).astype(np.float32), "bf16")
    r = _round16(rng.standard_normal((9, 128)).astype(np.float32), "bf16")
    w = _round16((1 + 0.1 * rng.standard_normal(128)).astype(np.float32), "bf16")
    a = orc.sum_add_rmsnorm("bf16", [x], r, w, 1e-6, fp8_mode=O.FP8_DYNAMIC)
    b = orc.add_rmsnorm("bf16", x, r, w, 1e-6, fp8_mode=O.FP8_DYNAMIC)
    for k in ("r16", "y16", "q", "scales"):
        assert np.array_equal(a[k], b[k]), k
