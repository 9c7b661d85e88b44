"""Pins of the oracle's e4m3 GEMM: exact integer products against numpy's
integer matmul, decoded products against numpy's float64 matmul (library
routines the oracle does not call), scale placement, transposition and
stride checks."""
import numpy as np
import pytest
import torch



def _codes(vals):
    """float values -> e4m3 codes via torch's cast (exact for grid values)."""
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def test_small_integers_exact(orc):
    """Integers -8..8 are exact e4m3 values; their products and sums are
    exact in fp64, so C equals numpy's integer matmul."""
    rng = np.random.default_rng(80)
    a_int = rng.integers(-8, 9, (5, 64))
    b_int = rng.integers(-8, 9, (7, 64))
    r = orc.fp8_gemm(_codes(a_int), 1.0, _codes(b_int), 1.0)
    assert np.array_equal(r["c"], (a_int @ b_int.T).astype(np.float64))


def test_random_codes_match_numpy(orc):
    rng = np.random.default_rng(81)
    a = rng.integers(0, 256, (6, 300)).astype(np.uint8)
    b = rng.integers(0, 256, (9, 300)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0   # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0
    sa = rng.uniform(0.1, 2, 6).astype(np.float32)
    sb = rng.uniform(0.1, 2, 9).astype(np.float32)
    r = orc.fp8_gemm(a, sa, b, sb)
    ref = sa[:, None].astype(np.float64) * (_dec(a) @ _dec(b).T) * sb[None, :].astype(np.float64)
    assert np.allclose(r["c"], ref, rtol=1e-12, atol=1e-12 * np.max(np.abs(ref)))


def test_scales_per_row_and_per_tensor(orc):
    a = _codes(np.ones((3, 32)))
    b = _codes(np.ones((4, 32)))
    r = orc.fp8_gemm(a, np.array([1, 2, 4], np.float32), b, np.array([1, 0.5, 0.25, 8], np.float32))
    assert np.array_equal(r["c"], 32.0 * np.outer([1, 2, 4], [1, 0.5, 0.25, 8]))
    r1 = orc.fp8_gemm(a, 2.0, b, 3.0)
    assert np.all(r1["c"] == 32 * 6.0)


def test_row_strides_and_k(orc):
    """Padded rows (ld > k) give the dense result; columns >= k are ignored."""
    rng = np.random.default_rng(82)
    a_int = rng.integers(-4, 5, (4, 48))
    b_int = rng.integers(-4, 5, (5, 48))
    a = np.full((4, 64), 0x7F, np.uint8)   # NaN padding
    b = np.full((5, 80), 0x7F, np.uint8)
    a[:, :48] = _codes(a_int)
    b[:, :48] = _codes(b_int)
    r = orc.fp8_gemm(a, 1.0, b, 1.0, k=48)
    assert np.array_equal(r["c"], (a_int @ b_int.T).astype(np.float64))


def test_c16_is_rne_of_c(orc):
    rng = np.random.default_rng(83)
    a = _codes(rng.standard_normal((3, 128)))
    b = _codes(rng.standard_normal((5, 128)))
    r = orc.fp8_gemm(a, 0.7, b, 1.3)
    ref = torch.from_numpy(r["c"]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch rounds float64 -> bf16 through float32 (double rounding); compare values
    back = torch.from_numpy(r["c16"].view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.all(np.abs(back - r["c"]) <= np.abs(r["c"]) * 2.0**-8)
    assert np.mean(r["c16"] == ref) > 0.99
