"""Pins of the fp64 oracle against things other than itself.

Each check compares the oracle with an independent source: a library's
conversion routine the oracle does not call (numpy float16, torch bfloat16,
torch float8_e4m3fn), the e4m3 bit identity printed in "MI210 LLM Stack"
(key insight 4), brute-force search, closed forms of the RMSNorm definition
(Zhang & Sennrich 2019, eq. 4), or invariants that definition implies.
"""
import math
import os
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _decode_all(orc, dtype):
    return np.array([orc.decode16(dtype, int(b)) for b in ALL16], np.float64)


# --------------------------------------------------------------------------
# 16-bit codecs
# --------------------------------------------------------------------------

def test_bf16_decode_matches_torch(orc):
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = _decode_all(orc, O.BF16)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_fp16_decode_matches_numpy(orc):
    ref = ALL16.view(np.float16).astype(np.float64)
    got = _decode_all(orc, O.FP16)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


@pytest.mark.parametrize("dtype", [O.BF16, O.FP16])
def test_encode16_round_trips_every_pattern(orc, dtype):
    vals = _decode_all(orc, dtype)
    for b, v in zip(ALL16, vals):
        if math.isnan(v):
            assert math.isnan(orc.decode16(dtype, orc.encode16(dtype, v)))
        else:
            assert orc.encode16(dtype, v) == b


@pytest.mark.parametrize("dtype", [O.BF16, O.FP16])
def test_encode16_midpoints_go_to_even(orc, dtype):
    """Between two adjacent finite patterns of one sign, the exact midpoint
    rounds to the pattern with an even last bit; a hair off the midpoint
    rounds to the nearer one."""
    vals = _decode_all(orc, dtype)
    inf_bits = 0x7F80 if dtype == O.BF16 else 0x7C00
    for sign in (0, 0x8000):
        lo_bits = np.arange(sign, sign + inf_bits - 1, 37, dtype=np.uint32)
        for b in lo_bits:
            a, c = vals[b], vals[b + 1]
            mid = (a + c) / 2.0  # exact: both have few significant bits
            even = b if b % 2 == 0 else b + 1
            assert orc.encode16(dtype, mid) == even
            toward_a = mid - (mid - a) * 2.0**-20
            toward_c = mid + (c - mid) * 2.0**-20
            assert orc.encode16(dtype, toward_a) == b
            assert orc.encode16(dtype, toward_c) == b + 1


@pytest.mark.parametrize("dtype", [O.BF16, O.FP16])
def test_encode16_overflow_edge(orc, dtype):
    maxb = 0x7F7F if dtype == O.BF16 else 0x7BFF
    inf_bits = 0x7F80 if dtype == O.BF16 else 0x7C00
    mx = orc.decode16(dtype, maxb)
    ulp = mx - orc.decode16(dtype, maxb - 1)
    assert orc.encode16(dtype, mx + ulp / 2) == inf_bits  # tie -> even -> Inf
    assert orc.encode16(dtype, mx + ulp / 2 * (1 - 2.0**-20)) == maxb
    assert orc.encode16(dtype, -(mx + ulp)) == 0x8000 | inf_bits
    assert orc.encode16(dtype, -0.0) == 0x8000


def test_fp16_encode_matches_numpy_on_random_doubles(orc):
    rng = np.random.default_rng(11)
    mant = rng.uniform(1.0, 2.0, 200_000)
    exps = rng.integers(-27, 17, 200_000)
    sign = np.where(rng.integers(0, 2, 200_000) == 1, -1.0, 1.0)
    v = sign * np.ldexp(mant, exps)
    with np.errstate(over="ignore"):  # overflow to +-Inf is part of the check
        ref = v.astype(np.float16).view(np.uint16)  # numpy rounds double -> half directly
    got = np.array([orc.encode16(O.FP16, float(a)) for a in v], np.uint16)
    assert np.array_equal(ref, got)


def test_bf16_encode_matches_torch_on_random_floats(orc):
    rng = np.random.default_rng(12)
    mant = rng.uniform(1.0, 2.0, 200_000)
    exps = rng.integers(-140, 128, 200_000)
    v = np.ldexp(mant, exps).astype(np.float32)  # torch converts from fp32
    v[::2] *= -1
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.encode16(O.BF16, float(a)) for a in v], np.uint16)
    assert np.array_equal(ref, got)


def _pairs(window):
    a = np.array(window, np.uint16)
    xs = np.repeat(a, len(a))
    rs = np.tile(a, len(a))
    return xs, rs


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("window", ["unit", "cancel", "subnormal"])
def test_residual_sum_equals_fp32_add_then_round(orc, dtype, window):
    """The stored residual: the oracle rounds the exact sum once; the GPU
    adds in fp32 and rounds to 16 bits.  fp32 has >= 2p+2 bits for both
    16-bit formats, so the double rounding is innocuous (Figueroa, "When is
    double rounding innocuous?", SIGNUM 1995) and the two rules agree on
    every pair.  Checked here against torch's / numpy's fp32 arithmetic on
    structured windows dense in rounding ties."""
    base = {"bf16": 0x3F00, "fp16": 0x3800}[dtype]
    if window == "unit":
        xs, rs = _pairs(range(base, base + 1024))
    elif window == "cancel":
        xs, rs = _pairs(range(base, base + 1024))
        rs = rs | 0x8000
    else:
        xs, rs = _pairs(range(0, 1024))
        rs = rs ^ np.where(np.arange(len(rs)) % 3 == 0, 0x8000, 0).astype(np.uint16)
    x2 = xs.reshape(1024, 1024)
    r2 = rs.reshape(1024, 1024)
    got = orc.add_rmsnorm(dtype, x2, r2, None, 1e-6, want_y=False)["r16"]
    if dtype == "bf16":
        tx = torch.from_numpy(x2.view(np.int16).copy()).view(torch.bfloat16).float()
        tr = torch.from_numpy(r2.view(np.int16).copy()).view(torch.bfloat16).float()
        ref = (tx + tr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        ref = (x2.view(np.float16).astype(np.float32) + r2.view(np.float16).astype(np.float32)
               ).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def _fp32_add_round16(dtype, xs, rs):
    """What the GPU does: decode both to fp32 exactly, add in fp32 (round
    to nearest even), round the fp32 sum to the 16-bit format (nearest
    even).  numpy's own fp32 arithmetic and fp32 -> fp16 conversion; the
    fp32 -> bf16 rounding by the bit rule for nearest-even on the upper 16
    bits of the fp32 pattern.  Returns the 16-bit patterns and a NaN mask."""
    if dtype == "fp16":
        s = xs.view(np.float16).astype(np.float32) + rs.view(np.float16).astype(np.float32)
        return s.astype(np.float16).view(np.uint16), np.isnan(s)
    s = ((xs.astype(np.uint32) << 16).view(np.float32)
         + (rs.astype(np.uint32) << 16).view(np.float32))
    u = s.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    return out, np.isnan(s)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_residual_sum_exhaustive(orc, dtype):
    """Every one of the 2^32 (x, residual) pairs of 16-bit patterns: the
    oracle's stored residual (exact sum, one rounding) equals fp32 add then
    16-bit rounding, bit for bit (NaN matches NaN).  This is the double-
    rounding theorem checked by brute force over the whole input space."""
    from concurrent.futures import ThreadPoolExecutor

    allv = np.arange(65536, dtype=np.uint16)
    chunk = 64

    def check(lo):
        xs = np.repeat(allv[lo:lo + chunk], 65536)
        rs = np.tile(allv, chunk)
        got = orc.residual16(dtype, xs, rs)
        with np.errstate(over="ignore", invalid="ignore"):
            ref, nan = _fp32_add_round16(dtype, xs, rs)
        if dtype == "fp16":
            got_nan = (got & 0x7C00) == 0x7C00
            got_nan &= (got & 0x03FF) != 0
        else:
            got_nan = ((got & 0x7F80) == 0x7F80) & ((got & 0x007F) != 0)
        bad = (got_nan != nan) | (~nan & (got != ref))
        return int(np.count_nonzero(bad)), (int(xs[bad][0]), int(rs[bad][0])) if bad.any() else None

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        results = list(ex.map(check, range(0, 65536, chunk)))
    nbad = sum(r[0] for r in results)
    first = next((r[1] for r in results if r[1]), None)
    assert nbad == 0, f"{nbad} pairs differ; first (x, res) = {first}"


# --------------------------------------------------------------------------
# OCP e4m3
# --------------------------------------------------------------------------

ALL8 = np.arange(256, dtype=np.uint16)


def test_e4m3_decode_matches_page_bit_identity(orc):
    """MI210 LLM Stack, key insight 4: h = ((u & 0x80) << 8) | ((u & 0x7f) << 7)
    is an fp16 holding exactly 2^-8 times the e4m3 value, for all 254
    non-NaN patterns."""
    h = ((ALL8 & 0x80) << 8) | ((ALL8 & 0x7F) << 7)
    via_fp16 = h.astype(np.uint16).view(np.float16).astype(np.float64) * 2.0**8
    finite = 0
    for u in range(256):
        v = orc.e4m3_decode(u)
        if (u & 0x7F) == 0x7F:
            assert math.isnan(v)
            continue
        finite += 1
        assert v == via_fp16[u]
        assert math.copysign(1.0, v) == math.copysign(1.0, via_fp16[u])
    assert finite == 254


def test_e4m3_decode_matches_torch(orc):
    t = torch.from_numpy(ALL8.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    for u in range(256):
        v = orc.e4m3_decode(u)
        assert (math.isnan(v) and math.isnan(t[u])) or v == t[u]
    assert orc.e4m3_decode(0x7E) == 448.0
    assert orc.e4m3_decode(0x01) == 2.0**-9


def _finite_codes(orc):
    codes = [u for u in range(256) if (u & 0x7F) != 0x7F]
    return codes, np.array([orc.e4m3_decode(u) for u in codes])


def _brute_e4m3(codes, vals, v):
    """Nearest finite code by exhaustive search; ties to the even mantissa;
    the sign of zero follows v; beyond 448 saturate."""
    if math.isnan(v):
        return 0x7F
    if abs(v) >= 448:
        return 0xFE if v < 0 else 0x7E
    d = np.abs(vals - v)
    best = np.flatnonzero(d == d.min())
    cands = [codes[i] for i in best]
    if v == 0 or all(vals[i] == 0 for i in best):
        return 0x80 if math.copysign(1.0, v) < 0 else 0x00
    cands = [c for c in cands if (c & 0x80) == (0x80 if v < 0 else 0)]
    if len(cands) > 1:
        cands = [c for c in cands if c % 2 == 0]
    assert len(cands) == 1
    return cands[0]


def test_e4m3_encode_brute_force(orc):
    codes, vals = _finite_codes(orc)
    pos = np.unique(vals[vals >= 0])
    sweep = list(pos)
    for a, b in zip(pos[:-1], pos[1:]):
        m = (a + b) / 2
        sweep += [m, np.nextafter(m, -1.0), np.nextafter(m, 2.0 * m + 1), a + (b - a) * 0.3]
    sweep += [448 * (1 + 2.0**-12), 460.0, 464.0, 1e30, math.inf, 2.0**-12, 2.0**-10,
              3 * 2.0**-11]
    rng = np.random.default_rng(5)
    sweep += list(np.ldexp(rng.uniform(1, 2, 3000), rng.integers(-12, 10, 3000)))
    for v in sweep:
        for s in (1.0, -1.0):
            assert orc.e4m3_encode(s * v) == _brute_e4m3(codes, vals, s * v), (s * v)
    assert orc.e4m3_encode(math.nan) == 0x7F
    assert orc.e4m3_encode(-0.0) == 0x80
    assert orc.e4m3_encode(-math.inf) == 0xFE


def test_e4m3_encode_matches_torch_in_range(orc):
    """torch's float -> float8_e4m3fn cast rounds to nearest even; in the
    finite range (|v| <= 448) it must agree with the saturating encoder."""
    rng = np.random.default_rng(6)
    v = np.ldexp(rng.uniform(1, 2, 100_000), rng.integers(-12, 9, 100_000)).astype(np.float32)
    v[::2] *= -1
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(a)) for a in v], np.uint8)
    assert np.array_equal(ref, got)


# --------------------------------------------------------------------------
# The RMSNorm definition
# --------------------------------------------------------------------------

def _bits(vals, dtype="bf16"):
    f = np.asarray(vals, np.float32)
    if dtype == "fp16":
        return f.astype(np.float16).view(np.uint16)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_hidden1_eps0_is_sign_times_weight(orc):
    for v, w in [(3.0, 1.5), (-0.25, 2.0), (1e-3, -0.5)]:
        r = orc.add_rmsnorm("bf16", _bits([[v]]), None, _bits([w]), 0.0)
        assert r["y"][0, 0] == math.copysign(1.0, v) * float(_bits_val([w]))


def _bits_val(vals):
    return torch.from_numpy(_bits(vals).view(np.int16)).view(torch.bfloat16).double().numpy()[0]


def test_three_four_row(orc):
    """H = 2, r = (3, 4): mean square 12.5, y = (3, 4) / sqrt(12.5)
    = (0.6, 0.8) * sqrt(2)."""
    r = orc.add_rmsnorm("fp16", _bits([[3.0, 4.0]], "fp16"), None, None, 0.0)
    assert r["y"][0, 0] == pytest.approx(0.6 * math.sqrt(2), rel=1e-15)
    assert r["y"][0, 1] == pytest.approx(0.8 * math.sqrt(2), rel=1e-15)


def test_fused_add_three_four(orc):
    """x + residual = (1 + 2, 5 - 1) = (3, 4) with weight (2, 0.5)."""
    r = orc.add_rmsnorm("bf16", _bits([[1.0, 5.0]]), _bits([[2.0, -1.0]]), _bits([2.0, 0.5]), 0.0)
    assert list(r["r16"][0]) == list(_bits([3.0, 4.0]))
    assert r["y"][0, 0] == pytest.approx(2 * 0.6 * math.sqrt(2), rel=1e-15)
    assert r["y"][0, 1] == pytest.approx(0.5 * 0.8 * math.sqrt(2), rel=1e-15)


def test_single_spike_pins_divisor_and_index(orc):
    """One nonzero entry a at column k of H: mean square a^2 / H, so
    y_k = sqrt(H) * w_k (eps = 0) and every other y is 0.  A divisor other
    than H (the row stride, H - 1) or a shifted index fails."""
    H, stride, k = 96, 128, 37
    x = np.zeros((1, stride), np.uint16)
    x[0, H:] = 0x7FA5  # NaN padding that must never be read
    x[0, k] = _bits([-5.0])[0]
    w = _bits(np.linspace(0.5, 1.5, H))
    r = orc.add_rmsnorm("bf16", x, None, w, 0.0, hidden=H)
    wk = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()[k]
    assert r["y"][0, k] == pytest.approx(-math.sqrt(H) * wk, rel=1e-15)
    others = np.delete(r["y"][0], k)
    assert np.all(others == 0)


def test_constant_row(orc):
    """r_j = c for all j: y_j = c / sqrt(c^2 + eps) * w_j."""
    c, eps, H = 0.75, 0.25, 64
    x = _bits(np.full((3, H), c))
    r = orc.add_rmsnorm("bf16", x, None, None, eps)
    assert np.allclose(r["y"], c / math.sqrt(c * c + eps), rtol=1e-15, atol=0)


def test_output_rms_is_one_and_eps_enters_inside_sqrt(orc):
    rng = np.random.default_rng(3)
    H = 1000
    x = _bits(rng.standard_normal((8, H)) * 0.01)
    r0 = orc.add_rmsnorm("bf16", x, None, None, 0.0)
    rms = np.sqrt(np.mean(r0["y"] ** 2, axis=1))
    assert np.allclose(rms, 1.0, rtol=1e-13)
    eps = 1e-4
    r1 = orc.add_rmsnorm("bf16", x, None, None, eps)
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    ms = np.mean(xv ** 2, axis=1)
    assert np.allclose(np.mean(r1["y"] ** 2, axis=1), ms / (ms + np.float32(eps)), rtol=1e-13)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_scale_invariance_and_odd_symmetry(orc, dtype):
    rng = np.random.default_rng(4)
    x = _bits(rng.standard_normal((4, 300)), dtype)
    w = _bits(1 + 0.1 * rng.standard_normal(300), dtype)
    base = orc.add_rmsnorm(dtype, x, None, w, 0.0)["y"]
    vals = x.view(np.float16).astype(np.float32) if dtype == "fp16" else \
        torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()
    for k in (-3, 2, 5):
        scaled = _bits(vals * np.float32(2.0**k), dtype)
        assert np.array_equal(orc.add_rmsnorm(dtype, scaled, None, w, 0.0)["y"], base)
    neg = x ^ np.uint16(0x8000)
    assert np.array_equal(orc.add_rmsnorm(dtype, neg, None, w, 0.0)["y"], -base)


def test_weight_multiplies_each_channel(orc):
    rng = np.random.default_rng(8)
    x = _bits(rng.standard_normal((3, 257)))
    w = _bits(rng.uniform(0.5, 1.5, 257))
    wv = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()
    y1 = orc.add_rmsnorm("bf16", x, None, None, 1e-6)["y"]
    yw = orc.add_rmsnorm("bf16", x, None, w, 1e-6)["y"]
    assert np.allclose(yw, y1 * wv[None, :], rtol=2e-16, atol=0)


def test_fused_equals_plain_on_rounded_sum(orc):
    rng = np.random.default_rng(9)
    x = _bits(rng.standard_normal((5, 513)))
    res = _bits(rng.standard_normal((5, 513)))
    w = _bits(rng.uniform(0.5, 1.5, 513))
    fused = orc.add_rmsnorm("bf16", x, res, w, 1e-5)
    plain = orc.add_rmsnorm("bf16", fused["r16"], None, w, 1e-5)
    assert np.array_equal(fused["y"], plain["y"])
    assert np.array_equal(fused["y16"], plain["y16"])


def test_strided_rows_never_read_padding(orc):
    rng = np.random.default_rng(10)
    H, S = 100, 128
    x = np.full((6, S), 0x7FA5, np.uint16)
    res = np.full((6, S), 0x7FA5, np.uint16)
    x[:, :H] = _bits(rng.standard_normal((6, H)))
    res[:, :H] = _bits(rng.standard_normal((6, H)))
    r = orc.add_rmsnorm("bf16", x, res, None, 1e-6, hidden=H)
    dense = orc.add_rmsnorm("bf16", x[:, :H].copy(), res[:, :H].copy(), None, 1e-6)
    assert np.all(np.isfinite(r["y"]))
    assert np.array_equal(r["y"], dense["y"])


def test_eps0_zero_row_is_nan(orc):
    r = orc.add_rmsnorm("bf16", np.zeros((1, 8), np.uint16), None, None, 0.0)
    assert np.all(np.isnan(r["y"]))


# --------------------------------------------------------------------------
# FP8 outputs
# --------------------------------------------------------------------------

def test_fp8_static_exact_points_and_saturation(orc):
    """x = 1 everywhere and eps = 0 make inv = 1, so y = w exactly and
    q = E(w / s).  With s a power of two and w on the e4m3 grid times s,
    the code is exact; w / s beyond 448 saturates to 0x7E / 0xFE."""
    codes, vals = _finite_codes(orc)
    grid = [v for v in vals if v != 0 and abs(v) <= 448][:200]
    s = 2.0**-3
    H = len(grid) + 2
    w = _bits(list(np.array(grid) * s) + [600 * s, -1000 * s])
    x = _bits(np.ones((1, H)))
    r = orc.add_rmsnorm("bf16", x, None, w, 0.0, fp8_mode=O.FP8_STATIC, static_scale=s)
    for j, v in enumerate(grid):
        assert orc.e4m3_decode(int(r["q"][0, j])) == v
    assert r["q"][0, H - 2] == 0x7E and r["q"][0, H - 1] == 0xFE


def test_fp8_dynamic_invariants(orc):
    rng = np.random.default_rng(13)
    H = 777
    x = _bits(rng.standard_normal((16, H)))
    x[3] = 0  # an all-zero row
    res = _bits(rng.standard_normal((16, H)))
    res[3] = 0
    w = _bits(1 + 0.1 * rng.standard_normal(H))
    r = orc.add_rmsnorm("bf16", x, res, w, 1e-6, fp8_mode=O.FP8_DYNAMIC)
    dec = np.vectorize(orc.e4m3_decode)(r["q"].astype(np.int64))
    for i in range(16):
        y = r["y"][i]
        amax = np.max(np.abs(y))
        if i == 3:
            assert amax == 0 and r["scales"][i] == 0 and np.all(r["q"][i] == 0)
            continue
        assert r["scales"][i] == np.float32(amax / 448)
        k = int(np.argmax(np.abs(y)))
        assert r["q"][i, k] & 0x7F == 0x7E  # the largest |y| maps to 448
        # RNE: |q*scale - y| <= half the e4m3 spacing at |y/scale| (the
        # slack covers only the fp64 rounding of the quotient itself).
        v = y / r["scales"][i]
        spacing = np.where(np.abs(v) < 2.0**-6, 2.0**-9,
                           np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(v), 1e-300))).astype(int) - 3))
        assert np.all(np.abs(dec[i] - v) <= spacing / 2 * (1 + 2.0**-40))


def test_fp8_static_code_decided_on_the_exact_quotient(orc):
    """x = 1, w = 1 and eps = 0 give y = 1 exactly, so the code is E(1 / s).
    With the fp32 scale s = 0.84210527, 1 / s = 1.18749999115..., just below
    the e4m3 tie 1.1875 between 1.125 (0x39) and 1.25 (0x3A): the nearest
    code is 0x39.  The same quotient rounded to fp32 first is the tie itself
    and would go to the even code 0x3A, so this pins the decision to the
    unrounded quotient."""
    s = np.float32(0.84210527)
    q = Fraction(1) / Fraction(float(s))
    tie = Fraction(19, 16)
    assert tie - Fraction(1, 2**24) < q < tie          # inside an fp32 half-ulp
    assert np.float32(1.0) / s == np.float32(1.1875)   # fp32 lands on the tie
    for dtype in ("bf16", "fp16"):
        r = orc.add_rmsnorm(dtype, _bits(np.ones((2, 8)), dtype), None,
                            _bits(np.ones(8), dtype), 0.0,
                            fp8_mode=O.FP8_STATIC, static_scale=float(s))
        assert np.all(r["y"] == 1.0)
        assert np.all(r["q"] == 0x39), r["q"]


def test_fp8_dynamic_code_decided_on_the_exact_quotient(orc):
    """Row (448, 17), eps = 0: y = r / rms, amax = 448 / rms and the stored
    scale is fp32(amax / 448) = fp32(1 / rms).  The second code is
    E(17 (1 / rms) / scale): computed to 60 digits the quotient lies 1.9e-7
    above the tie 17 between 16 (0x58) and 18 (0x59), so the nearest code
    is 0x59.  Rounded to fp32 first it would be 17 itself and go to the
    even 0x58."""
    with localcontext() as ctx:
        ctx.prec = 60
        rms = ((Decimal(448) ** 2 + Decimal(17) ** 2) / 2).sqrt()
        scale = np.float32(float(1 / rms))
        q = Decimal(17) / rms / Decimal(float(scale))
        assert Decimal(0) < q - 17 < Decimal(2.0**-20)  # above the tie, inside an fp32 half-ulp
        assert np.float32(float(q)) == np.float32(17.0)
    r = orc.add_rmsnorm("bf16", _bits([[448.0, 17.0]]), None, None, 0.0,
                        fp8_mode=O.FP8_DYNAMIC)
    assert r["scales"][0] == scale
    assert r["q"][0, 0] == 0x7E and r["q"][0, 1] == 0x59, r["q"]


def test_fp8_dynamic_zero_row_only(orc):
    r = orc.add_rmsnorm("fp16", np.zeros((2, 64), np.uint16), None, None, 1e-5,
                        fp8_mode=O.FP8_DYNAMIC)
    assert np.all(r["scales"] == 0) and np.all(r["q"] == 0)


def test_fp8_dynamic_scales_beyond_fp32(orc):
    """The stored scale is fp32(amax / 448) and the codes are E(y / scale)
    against that stored value, wherever it lands:
      * x = w = 2^-133 (bf16's smallest subnormal), eps = 1e-6: amax is
        about 2^-256, the scale rounds to 0, y / 0 is +-inf and saturates to
        +-448 (0x7E / 0xFE), and an exact zero gives 0 / 0, the NaN code;
      * x = 1, w = 2^-130, eps = 0: y = w exactly, amax / 448 = 2^-138.807
        rounds to the fp32 subnormal 1170 * 2^-149, and y / scale =
        2^19 / 1170 = 448.109..., which still rounds to 448;
      * with the variance over the first channel only, r = (2^-60, 2^100,
        -2^100, 3), eps = 0: y_1 = 2^160, amax / 448 exceeds fp32's range,
        the scale is +inf and every code is E(y / inf) = +-0."""
    b = lambda a: _bits(np.asarray(a, np.float64))
    t = 2.0**-133
    r = orc.add_rmsnorm("bf16", b([[t, -t, 0.0, t]]), None, b([t] * 4), 1e-6,
                        fp8_mode=O.FP8_DYNAMIC)
    assert r["scales"][0] == 0 and 0 < np.max(np.abs(r["y"][0])) < 2.0**-250
    assert list(r["q"][0, [0, 1, 3]]) == [0x7E, 0xFE, 0x7E]
    assert r["q"][0, 2] & 0x7F == 0x7F
    r = orc.add_rmsnorm("bf16", b([[1.0] * 8]), None, b([2.0**-130] * 8), 0.0,
                        fp8_mode=O.FP8_DYNAMIC)
    assert np.all(r["y"][0] == 2.0**-130)
    assert r["scales"][0] == np.float32(1170 * 2.0**-149)
    assert Fraction(2**19, 1170) == Fraction(2.0**-130) / Fraction(1170 * 2.0**-149)
    assert np.all(r["q"][0] == 0x7E)
    r = orc.add_rmsnorm("bf16", b([[2.0**-60, 2.0**100, -2.0**100, 3.0]]), None, None, 0.0,
                        fp8_mode=O.FP8_DYNAMIC, variance_size=1)
    assert r["y"][0, 1] == 2.0**160 and np.isinf(r["scales"][0]) and r["scales"][0] > 0
    assert list(r["q"][0]) == [0x00, 0x00, 0x80, 0x00]


def test_variance_size_override_closed_form(orc):
    """variance_size = k: the mean square of the first k channels
    normalises every channel.  Row (a, .., a | b, .., b) with k a's gives
    y = r / sqrt(a^2 + eps)."""
    H, k, a, b, eps = 64, 24, 0.5, 3.0, 0.25
    x = _bits([[a] * k + [b] * (H - k)])
    r = orc.add_rmsnorm("bf16", x, None, None, eps, variance_size=k)
    assert np.allclose(r["y"][0, :k], a / math.sqrt(a * a + eps), rtol=1e-15, atol=0)
    assert np.allclose(r["y"][0, k:], b / math.sqrt(a * a + eps), rtol=1e-15, atol=0)
    full = orc.add_rmsnorm("bf16", x, None, None, eps, variance_size=H)
    assert np.array_equal(full["y"], orc.add_rmsnorm("bf16", x, None, None, eps)["y"])
