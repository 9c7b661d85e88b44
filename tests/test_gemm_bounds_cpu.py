"""The GEMM tolerance's two sums (tests/_helpers.py gemm_bounds), checked
against plain loops.  They are test infrastructure, not part of the GEMM's
definition, so they live beside the tests rather than in the oracle."""
import numpy as np
import torch

from tests._helpers import e4m3_values, gemm_bounds


def _codes(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_abs_sum_on_integers():
    rng = np.random.default_rng(80)
    a_int = rng.integers(-8, 9, (5, 64))
    b_int = rng.integers(-8, 9, (7, 64))
    absum, _ = gemm_bounds(_codes(a_int), 1.0, _codes(b_int), 1.0, 64)
    assert np.array_equal(absum, (np.abs(a_int) @ np.abs(b_int).T).astype(np.float64))


def test_stepmax_against_loops():
    """Per output, the sum over 128-wide k steps (the last one partial) of
    the largest |product|, times |sa sb|; per-row and per-tensor scales."""
    rng = np.random.default_rng(12)
    m, n, k = 3, 5, 300
    a = _codes(np.clip(rng.standard_normal((m, k)) * 8, -448, 448))
    b = _codes(np.clip(rng.standard_normal((n, k)) * 2, -448, 448))
    sa = rng.uniform(0.5, 2, m).astype(np.float32)
    sb = np.array([0.25], np.float32)
    absum, step = gemm_bounds(a, sa, b, sb, k)
    da, db = e4m3_values(a), e4m3_values(b)
    for i in range(m):
        for j in range(n):
            p = np.abs(da[i] * db[j])
            want = sum(p[s:s + 128].max() for s in range(0, k, 128)) * float(sa[i]) * 0.25
            assert step[i, j] == want
            assert abs(absum[i, j] - p.sum() * float(sa[i]) * 0.25) <= 1e-12 * absum[i, j]
    assert np.all(step <= absum)


def test_columns_past_k_ignored():
    a = np.full((2, 160), 0x7E, np.uint8)   # 448 past k
    b = np.full((3, 160), 0x7E, np.uint8)
    a[:, :130] = _codes(np.ones((2, 130)))
    b[:, :130] = _codes(np.full((3, 130), 2.0))
    absum, step = gemm_bounds(a, np.float32(1), b, np.float32(1), 130)
    assert np.all(absum == 260.0) and np.all(step == 4.0)
