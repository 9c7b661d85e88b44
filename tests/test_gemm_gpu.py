"""Parity of the e4m3 skinny GEMM (MFMA path, through the C ABI) with the
oracle.

Tolerance (tests/_helpers.py gemm_tol): the oracle sums in fp64; the GPU's
matrix unit keeps about 13 bits below the largest product of each 128-wide
k step, the steps and waves are summed in fp32, and the result is rounded
once to 16 bits:
    |c - c_ref| <= rho |c_ref| + ulp16(c_ref) + 2^-8 stepmax_ref
                   + (k/128 + 256) 2^-24 abs_ref.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests._helpers import bits, dev, gemm_ref, gemm_tol, values16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _codes(rng, rows, cols, std):
    f = torch.from_numpy((rng.standard_normal((rows, cols)) * std).astype(np.float32))
    return f.clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check(orc, m, n, k, out="bf16", per_row=(True, True), seed=0, lda=None, ldb=None,
          pre=False, workspace=None, repeat=1):
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(seed)
    lda, ldb = lda or k, ldb or k
    a = np.full((m, lda), 0x7F, np.uint8)   # NaN codes in any padding
    b = np.full((n, ldb), 0x7F, np.uint8)
    a[:, :k] = _codes(rng, m, k, 24.0)
    b[:, :k] = _codes(rng, n, k, 6.0)
    sa = rng.uniform(0.01, 0.1, m if per_row[0] else 1).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n if per_row[1] else 1).astype(np.float32)
    ad = torch.from_numpy(a).cuda()[:, :k]
    bd = torch.from_numpy(b).cuda()[:, :k]
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[out]
    c = torch.full((m + 1, n), float("nan"), dtype=dt, device="cuda")
    if pre:
        bd = arn.fp8_weight_preshuffle(bd)
    sad, sbd = torch.from_numpy(sa).cuda(), torch.from_numpy(sb).cuda()
    arn.fp8_gemm(ad, sad, bd, sbd, out=c[:m], workspace=workspace)
    first = c[:m].clone()
    for _ in range(repeat - 1):   # the workspace is left ready for the next call
        arn.fp8_gemm(ad, sad, bd, sbd, out=c[:m], workspace=workspace)
        assert torch.equal(c[:m], first), "repeated call differs"
    torch.cuda.synchronize()
    ref = gemm_ref(orc, a, sa if per_row[0] else sa[0], b, sb if per_row[1] else sb[0], k=k,
                       out_dtype=out)
    got = values16(bits(c[:m]), out)
    tol = gemm_tol(ref, k, out)
    err = np.abs(got - ref["c"])
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol)} at {np.unravel_index(np.argmax(err / tol), err.shape)}"
    assert torch.isnan(c[m].float()).all(), "wrote past the last row"
    return arn.last_plan()


LAYOUTS = pytest.mark.parametrize("pre", [False, True], ids=["rowmajor", "preshuffled"])


@LAYOUTS
@pytest.mark.parametrize("m", [1, 2, 7, 16, 17, 32, 33, 64])
def test_rows(orc, m, pre):
    check(orc, m, 200, 1024, seed=m, pre=pre)


@LAYOUTS
@pytest.mark.parametrize("n,k", [(1, 32), (16, 16), (33, 48), (63, 96), (64, 128), (100, 160),
                                 (70, 208), (517, 2048),
                                 (1000, 4096), (2304, 16384), (13312, 512)])
def test_shapes(orc, n, k, pre):
    check(orc, 4, n, k, seed=n + k, pre=pre)


@LAYOUTS
@pytest.mark.parametrize("m", [1, 8])
def test_logged_decode_shape(orc, m, pre):
    """The decode fp8 GEMM shape in the AITER log of "VLLM_ROCM_USE_AITER=1
    slows Gemma 4 on an AMD MI300X" (section "Why the fp8 Multiplies Run
    Slower": M 1, N 8192, K 3840, a pre-shuffled e4m3 weight), at M = 1 and 8."""
    check(orc, m, 8192, 3840, seed=100 + m, pre=pre)


@LAYOUTS
@pytest.mark.parametrize("per_row", [(False, False), (True, False), (False, True)])
def test_scale_modes(orc, per_row, pre):
    check(orc, 5, 300, 640, per_row=per_row, seed=3, pre=pre)


@LAYOUTS
def test_fp16_out(orc, pre):
    check(orc, 8, 512, 2048, out="fp16", seed=4, pre=pre)


@LAYOUTS
def test_padded_rows(orc, pre):
    """Row strides past K hold NaN codes that must never be read."""
    check(orc, 6, 130, 1040, lda=1056, ldb=1072, seed=5, pre=pre)


@pytest.mark.parametrize("cfg", [(1, 4), (1, 8), (1, 16), (2, 4), (2, 8), (2, 16), (4, 4),
                                 (4, 8), (4, 16)])
@pytest.mark.parametrize("m", [3, 20, 40])
def test_forced_configs(orc, m, cfg):
    """Every compiled block shape that the row tiling has, both layouts."""
    import residual_add_rmsnorm_amd as arn

    mt = 1 if m <= 16 else (2 if m <= 32 else 4)
    arn.set_gemm_config(*cfg)
    try:
        for pre in (False, True):
            try:
                plan = check(orc, m, 330, 1296, seed=m + cfg[0], pre=pre)
            except arn.ArnError as e:
                assert e.status == 2   # shape not compiled for this row tiling
                continue
            assert f"mt{mt}/nt{cfg[0]}/waves{cfg[1]}/" in plan
    finally:
        arn.set_gemm_config(0, 0)


def test_preshuffled_size():
    import residual_add_rmsnorm_amd as arn

    w = arn.fp8_weight_preshuffle(torch.zeros(33, 208, dtype=torch.uint8, device="cuda"))
    assert w.data.numel() == 3 * 2 * 2048 and w.shape == (33, 208)


def test_preshuffle_unaligned_weight(orc):
    """The shuffle reads any row stride; the GEMM then serves a weight whose
    own rows are not 16-byte aligned (row-major arn_fp8_gemm refuses it)."""
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(11)
    m, n, k, ldb = 3, 90, 336, 345
    a = _codes(rng, m, k, 24.0)
    b = np.full((n * ldb + 1,), 0x7F, np.uint8)
    bv = b[1:].reshape(n, ldb)            # odd base address, odd stride
    bv[:, :k] = _codes(rng, n, k, 6.0)
    sa = np.full(m, 0.05, np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    bd = torch.from_numpy(b).cuda()[1:].view(n, ldb)[:, :k]
    ad, sad, sbd = (torch.from_numpy(x).cuda() for x in (a, sa, sb))
    with pytest.raises(arn.ArnError):
        arn.fp8_gemm(ad, sad, bd, sbd)
    c = arn.fp8_gemm(ad, sad, arn.fp8_weight_preshuffle(bd), sbd)
    ref = gemm_ref(orc, a, sa, np.ascontiguousarray(bv[:, :k]), sb)
    got = values16(bits(c), "bf16")
    tol = gemm_tol(ref, k)
    assert np.all(np.abs(got - ref["c"]) <= tol)


@LAYOUTS
def test_nan_codes_propagate(orc, pre):
    """A NaN code (0x7F / 0xFF) inside K makes its whole output row (in A) or
    column (in B) NaN, as in the oracle's definition; every other output is
    unaffected.  (The rest of the suite keeps NaN codes in row padding,
    which must never be read.)"""
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(12)
    m, n, k = 5, 70, 640
    a = _codes(rng, m, k, 24.0)
    b = _codes(rng, n, k, 6.0)
    a[2, 300] = 0x7F
    b[41, 5] = 0xFF
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    bd = torch.from_numpy(b).cuda()
    if pre:
        bd = arn.fp8_weight_preshuffle(bd)
    ad, sad, sbd = (torch.from_numpy(x).cuda() for x in (a, sa, sb))
    c = arn.fp8_gemm(ad, sad, bd, sbd).float().cpu().numpy()
    ref = gemm_ref(orc, a, sa, b, sb)
    nan_ref = np.isnan(ref["c"])
    assert nan_ref[2].all() and nan_ref[:, 41].all() and nan_ref.sum() == n + m - 1
    assert np.array_equal(np.isnan(c), nan_ref)
    ok = ~nan_ref
    tol = gemm_tol({k2: (v[ok] if isinstance(v, np.ndarray) and v.shape == ref["c"].shape else v)
                    for k2, v in ref.items()}, k)
    assert np.all(np.abs(c[ok] - ref["c"][ok]) <= tol)


def test_deterministic():
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(6)
    a = torch.from_numpy(_codes(rng, 8, 4096, 24)).cuda()
    b = torch.from_numpy(_codes(rng, 2048, 4096, 6)).cuda()
    sa = torch.full((8,), 0.05, device="cuda")
    sb = torch.full((2048,), 0.004, device="cuda")
    r1 = arn.fp8_gemm(a, sa, b, sb)
    r2 = arn.fp8_gemm(a, sa, b, sb)
    bw = arn.fp8_weight_preshuffle(b)
    r3 = arn.fp8_gemm(a, sa, bw, sb)
    r4 = arn.fp8_gemm(a, sa, bw, sb)
    assert torch.equal(r1, r2)
    assert torch.equal(r3, r4)


def test_unsupported_shapes():
    import residual_add_rmsnorm_amd as arn

    a = torch.zeros(65, 128, dtype=torch.uint8, device="cuda")
    b = torch.zeros(64, 128, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, device="cuda")
    with pytest.raises(arn.ArnError) as e:
        arn.fp8_gemm(a, s, b, s)           # m > 64
    assert e.value.status == 2
    with pytest.raises(arn.ArnError) as e:
        arn.fp8_gemm(a[:4, :100], s, b[:, :100], s)   # k % 16 != 0
    assert e.value.status == 2


def test_swiglu_codes_feed_gemm(orc):
    """The decode pipeline: SwiGLU with dynamic e4m3 writes codes and
    per-row scales; the GEMM consumes them with a per-row-scaled weight.
    Both stages checked against the oracle run on the same data."""
    import residual_add_rmsnorm_amd as arn
    import workloads as W

    rng = np.random.default_rng(7)
    m, d, n = 8, 2048, 768
    x = W.to_bits((rng.standard_normal((m, 2 * d)) * 2).astype(np.float32), "bf16")
    q, sq = arn.silu_and_mul_fp8(dev(x, "bf16"), dynamic=True)
    b = _codes(rng, n, d, 6.0)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    c = arn.fp8_gemm(q, sq, torch.from_numpy(b).cuda(), torch.from_numpy(sb).cuda())
    torch.cuda.synchronize()
    qa = q.view(torch.uint8).cpu().numpy()
    sqa = sq.cpu().numpy()
    ref_g = orc.silu_and_mul("bf16", x, fp8_mode=O.FP8_DYNAMIC)
    # the GEMM is checked on the codes the GPU produced (those match the
    # oracle's within one step, checked by the SwiGLU tests)
    assert np.mean(qa == ref_g["q"]) > 0.99
    ref = gemm_ref(orc, qa, sqa, b, sb)
    got = values16(bits(c), "bf16")
    tol = gemm_tol(ref, d)
    assert np.all(np.abs(got - ref["c"]) <= tol)


@pytest.mark.parametrize("name", ["fp8_gemm_gate_up_13312x16384", "fp8_gemm_down_16384x6656",
                                  "fp8_gemm_qkv_2304x16384", "fp8_gemm_o_16384x2048"])
def test_full_size(orc, name):
    """The benchmark's GEMM shapes and data (the bench's generator), in its
    launch configuration (automatic block shape), both weight layouts, at
    M = 1 and 64: sampled output columns against the oracle computed on
    the matching weight rows."""
    import residual_add_rmsnorm_amd as arn
    import workloads as W

    g = W.GEMMS[name]
    print(f"\n[full-size] {name}", flush=True)
    d = W.make_gemm(g, 64)
    cols = np.unique(np.concatenate([np.linspace(0, g.n - 1, 160).astype(np.int64),
                                     [0, 15, 16, 63, 64, g.n // 2, g.n - 17, g.n - 16,
                                      g.n - 1]]))
    bd = torch.from_numpy(d["b"]).cuda()
    sbd = torch.from_numpy(d["scale_b"]).cuda()
    layouts = {"rowmajor": bd, "preshuffled": arn.fp8_weight_preshuffle(bd)}
    for m in (1, 64):
        a, sa = d["a"][:m], d["scale_a"][:m]
        ref = gemm_ref(orc, a, sa, np.ascontiguousarray(d["b"][cols]), d["scale_b"][cols])
        tol = gemm_tol(ref, g.k)
        ad, sad = torch.from_numpy(a).cuda(), torch.from_numpy(sa).cuda()
        for layout, b in layouts.items():
            c = arn.fp8_gemm(ad, sad, b, sbd)
            torch.cuda.synchronize()
            got = values16(bits(c[:, torch.from_numpy(cols).cuda()]), "bf16")
            err = np.abs(got - ref["c"])
            assert np.all(err <= tol), (m, layout, arn.last_plan(), float(np.max(err / tol)))
            assert torch.isfinite(c.float()).all(), (m, layout)



def test_preshuffled_panels(orc):
    """A weight whose pre-shuffled copy spans two panels: at K = 131072 a
    1 GiB panel holds 512 column tiles (8192 columns), and N = 8236 leaves
    a second panel of 4 tiles, the last one ragged.  Columns on both sides
    of the panel boundary and at the ragged end against the oracle, without
    and with a split-K workspace (3 splits forced)."""
    import residual_add_rmsnorm_amd as arn

    m, n, k = 3, 8236, 131072
    print(f"\n[panels] m {m} n {n} k {k}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(5)
    b = torch.randint(0, 256, (n, k), dtype=torch.uint8, device="cuda", generator=gen)
    b[(b & 0x7F) == 0x7F] = 0  # no NaN codes
    rng = np.random.default_rng(31)
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    cols = np.unique(np.concatenate([np.linspace(0, n - 1, 24).astype(np.int64),
                                     [0, 15, 16, 4095, 8175, 8176, 8191, 8192, 8207, 8208,
                                      8223, 8224, 8235]]))
    ref = gemm_ref(orc, a, sa, b[torch.from_numpy(cols).cuda()].cpu().numpy(), sb[cols])
    tol = gemm_tol(ref, k)
    pre = arn.fp8_weight_preshuffle(b)
    del b
    ad, sad, sbd = (torch.from_numpy(v).cuda() for v in (a, sa, sb))
    ws = arn.fp8_gemm_workspace(m, n, k)
    try:
        for splits, w in ((0, None), (3, ws)):
            arn.set_gemm_splits(splits)
            c = arn.fp8_gemm(ad, sad, pre, sbd, workspace=w)
            torch.cuda.synchronize()
            got = values16(bits(c[:, torch.from_numpy(cols).cuda()]), "bf16")
            err = np.abs(got - ref["c"])
            assert np.all(err <= tol), (splits, arn.last_plan(), float(np.max(err / tol)))
    finally:
        arn.set_gemm_splits(0)


def test_rowmajor_weight_past_2gib(orc):
    """A row-major weight over 2 GiB: a launch addresses at most 2 GiB of it
    (32-bit buffer offsets), so at K = 131072 the first launch takes 16384
    weight rows and a second one the last 116.  Columns on both sides of the
    launch boundary and at the end against the oracle, without and with a
    split-K workspace (3 splits forced: the second launch's partial tiles and
    counters start past the first launch's)."""
    import residual_add_rmsnorm_amd as arn

    m, n, k = 3, 16500, 131072
    assert n * k > 1 << 31
    print(f"\n[row-major past 2 GiB] m {m} n {n} k {k}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(6)
    b = torch.randint(0, 256, (n, k), dtype=torch.uint8, device="cuda", generator=gen)
    b[(b & 0x7F) == 0x7F] = 0  # no NaN codes
    rng = np.random.default_rng(32)
    a = rng.integers(0, 256, (m, k)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, n).astype(np.float32)
    cols = np.unique(np.concatenate([np.linspace(0, n - 1, 24).astype(np.int64),
                                     [0, 15, 16, 16367, 16368, 16383, 16384, 16385, 16399,
                                      16400, 16495, 16496, 16499]]))
    ref = gemm_ref(orc, a, sa, b[torch.from_numpy(cols).cuda()].cpu().numpy(), sb[cols])
    tol = gemm_tol(ref, k)
    ad, sad, sbd = (torch.from_numpy(v).cuda() for v in (a, sa, sb))
    ws = arn.fp8_gemm_workspace(m, n, k)
    try:
        for splits, w in ((0, None), (3, ws)):
            arn.set_gemm_splits(splits)
            c = arn.fp8_gemm(ad, sad, b, sbd, workspace=w)
            torch.cuda.synchronize()
            got = values16(bits(c[:, torch.from_numpy(cols).cuda()]), "bf16")
            err = np.abs(got - ref["c"])
            assert np.all(err <= tol), (splits, arn.last_plan(), float(np.max(err / tol)))
            assert "grid" in arn.last_plan()
    finally:
        arn.set_gemm_splits(0)
    assert _counters_zero(ws, n)


# ---------------------------------------------------------------------------
# Split K across blocks (workspace entry points)
# ---------------------------------------------------------------------------

def _counters_zero(ws, n):
    """The counter region is the tail of the workspace (its last
    ceil((size/512 + 1) / 256) * 256 bytes of the 256-byte-rounded size)."""
    usable = ws.numel() // 256 * 256
    cbytes = -(-(usable // 512 + 1) // 256) * 256
    return bool((ws[usable - cbytes:usable] == 0).all())


@LAYOUTS
@pytest.mark.parametrize("splits", [2, 3, 4, 8])
@pytest.mark.parametrize("m,n,k", [(1, 2304, 16384), (5, 300, 1040), (17, 130, 4096),
                                   (64, 1000, 2048), (3, 70, 256), (2, 64, 128)])
def test_split_k(orc, m, n, k, splits, pre):
    """Forced splits (capped by the k steps: k = 128 has one), each call
    checked against the oracle; the workspace is reused three times and its
    counters are zero afterwards."""
    import residual_add_rmsnorm_amd as arn

    ws = arn.fp8_gemm_workspace(m, n, k)
    arn.set_gemm_splits(splits)
    try:
        plan = check(orc, m, n, k, seed=m + n + splits, pre=pre, workspace=ws, repeat=3)
    finally:
        arn.set_gemm_splits(0)
    nsteps = (k + 127) // 128
    per = -(-nsteps // min(splits, nsteps))
    assert f"/splits{-(-nsteps // per)}/" in plan, plan
    torch.cuda.synchronize()
    assert _counters_zero(ws, n), "counters not reset"


@LAYOUTS
def test_split_k_auto_matches_oracle(orc, pre):
    import residual_add_rmsnorm_amd as arn

    for m, n, k in ((1, 2304, 16384), (16, 16384, 2048), (40, 520, 6656)):
        ws = arn.fp8_gemm_workspace(m, n, k)
        check(orc, m, n, k, seed=m, pre=pre, workspace=ws, repeat=2)
        assert _counters_zero(ws, n)


def test_split_k_many_calls_one_workspace(orc):
    """Back-to-back calls on one workspace, shapes alternating, each result
    equal to the first call of its shape (a counter left non-zero, or a
    partial read before it was written, would show up as a difference)."""
    import residual_add_rmsnorm_amd as arn

    rng = np.random.default_rng(21)
    shapes = [(1, 2304, 16384), (4, 4096, 2048), (33, 700, 1024)]
    ws = arn.fp8_gemm_workspace(64, 4096, 16384)
    data = []
    for m, n, k in shapes:
        a = torch.from_numpy(_codes(rng, m, k, 24.0)).cuda()
        b = arn.fp8_weight_preshuffle(torch.from_numpy(_codes(rng, n, k, 6.0)).cuda())
        sa = torch.full((m,), 0.05, device="cuda")
        sb = torch.full((n,), 0.004, device="cuda")
        data.append((a, sa, b, sb))
    arn.set_gemm_splits(4)
    try:
        firsts = [arn.fp8_gemm(*d, workspace=ws).clone() for d in data]
        for it in range(40):
            i = it % len(data)
            assert torch.equal(arn.fp8_gemm(*data[i], workspace=ws), firsts[i]), (it, shapes[i])
    finally:
        arn.set_gemm_splits(0)
    torch.cuda.synchronize()
    assert _counters_zero(ws, 4096)
    # and the split results agree with the unsplit kernel within the bound
    for (a, sa, b, sb), f in zip(data, firsts):
        ref = arn.fp8_gemm(a, sa, b, sb)
        assert torch.allclose(f.float(), ref.float(), rtol=2**-6, atol=1e-3)


def test_split_k_workspace_checks():
    import residual_add_rmsnorm_amd as arn
    from residual_add_rmsnorm_amd import _lib

    a = torch.zeros(4, 256, dtype=torch.uint8, device="cuda")
    b = torch.zeros(64, 256, dtype=torch.uint8, device="cuda")
    s = torch.ones(1, device="cuda")
    small = torch.zeros(_lib.load().arn_fp8_gemm_workspace_bytes(4, 64, 256) - 4,
                        dtype=torch.uint8, device="cuda")
    with pytest.raises(arn.ArnError) as e:
        arn.fp8_gemm(a, s, b, s, workspace=small)          # too small
    assert e.value.status == 1
    big = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    with pytest.raises(arn.ArnError) as e:
        arn.fp8_gemm(a, s, b, s, workspace=big[16:])       # not 256-byte aligned
    assert e.value.status == 1


# ---------------------------------------------------------------------------
# Exact cases: zero tolerance
# ---------------------------------------------------------------------------

def _exact_codes(rng, rows, cols):
    """Codes of the values k/4 with |k| <= 16, all exact e4m3.  Products are
    multiples of 2^-4 no larger than 16, so the sum of any 128-wide k step
    needs 8 bits below its largest product, and a whole row of K <= 16384
    stays within 2^18 on a 2^-4 grid (22 bits): every partial sum the matrix
    unit, the waves and the splits form is exact in fp32."""
    v = rng.integers(-16, 17, (rows, cols)).astype(np.float32) / 4
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def exact_data(m, n, k, per_row=(True, True), seed=0):
    rng = np.random.default_rng(1000 + seed)
    a = _exact_codes(rng, m, k)
    b = _exact_codes(rng, n, k)
    sa = np.ldexp(1.0, rng.integers(-3, 4, m if per_row[0] else 1)).astype(np.float32)
    sb = np.ldexp(1.0, rng.integers(-3, 4, n if per_row[1] else 1)).astype(np.float32)
    return a, sa, b, sb


def check_exact(orc, m, n, k, pre, out="bf16", per_row=(True, True), seed=0, workspace=None,
                cols=None, data=None):
    """c16 of the GPU equal to the oracle's bit for bit (power-of-two scales
    keep the scaled result exact too, so both sides round the same value
    once).  `cols` limits the comparison to sampled output columns."""
    import residual_add_rmsnorm_amd as arn

    assert k <= 16384
    a, sa, b, sb = data if data is not None else exact_data(m, n, k, per_row, seed)
    a = a[:m]
    sa = sa[:m] if sa.size > 1 else sa
    bd = torch.from_numpy(b).cuda()
    if pre:
        bd = arn.fp8_weight_preshuffle(bd)
    ad, sad, sbd = (torch.from_numpy(np.ascontiguousarray(v)).cuda() for v in (a, sa, sb))
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[out]
    c = torch.empty((m, n), dtype=dt, device="cuda")
    arn.fp8_gemm(ad, sad, bd, sbd, out=c, workspace=workspace)
    torch.cuda.synchronize()
    del bd
    got = bits(c)
    if cols is not None:
        b = np.ascontiguousarray(b[cols])
        sb = sb[cols] if sb.size > 1 else sb
        got = got[:, cols]
    ref = orc.fp8_gemm(a, sa if sa.size > 1 else sa[0], b, sb if sb.size > 1 else sb[0], k=k,
                       out_dtype=out)
    bad = np.flatnonzero(got != ref["c16"])
    assert bad.size == 0, (f"{bad.size} outputs differ; first at {np.unravel_index(bad[0], got.shape)}: "
                           f"gpu {got.ravel()[bad[0]]:#06x} ref {ref['c16'].ravel()[bad[0]]:#06x} "
                           f"({arn.last_plan()})")
    return arn.last_plan()


@LAYOUTS
@pytest.mark.parametrize("m,n,k", [(1, 200, 1024), (2, 70, 208), (8, 2304, 16384),
                                   (16, 517, 2048), (17, 1000, 4096), (33, 300, 640),
                                   (64, 2304, 2064), (1, 13312, 512)])
def test_gemm_exact_auto(orc, m, n, k, pre):
    check_exact(orc, m, n, k, pre, seed=m + n + k)


@LAYOUTS
@pytest.mark.parametrize("per_row", [(False, False), (True, False), (False, True)])
def test_gemm_exact_scale_modes_fp16(orc, per_row, pre):
    check_exact(orc, 5, 300, 640, pre, out="fp16", per_row=per_row, seed=7)


@pytest.mark.parametrize("cfg", [(1, 4), (1, 8), (1, 16), (2, 4), (2, 8), (2, 16), (4, 4),
                                 (4, 8), (4, 16)])
@pytest.mark.parametrize("m", [3, 20, 40])
def test_gemm_exact_forced_configs(orc, m, cfg):
    """Every compiled block shape of each row tiling, both layouts."""
    import residual_add_rmsnorm_amd as arn

    mt = 1 if m <= 16 else (2 if m <= 32 else 4)
    arn.set_gemm_config(*cfg)
    try:
        for pre in (False, True):
            try:
                plan = check_exact(orc, m, 330, 1296, pre, seed=m + cfg[0] + cfg[1])
            except arn.ArnError as e:
                assert e.status == 2   # shape not compiled for this row tiling
                continue
            assert f"mt{mt}/nt{cfg[0]}/waves{cfg[1]}/" in plan
    finally:
        arn.set_gemm_config(0, 0)


@LAYOUTS
@pytest.mark.parametrize("splits", [2, 3, 4, 8])
@pytest.mark.parametrize("m,n,k", [(1, 2304, 16384), (5, 300, 1040), (17, 130, 4096),
                                   (64, 1000, 2048)])
def test_gemm_exact_split_k(orc, m, n, k, splits, pre):
    import residual_add_rmsnorm_amd as arn

    ws = arn.fp8_gemm_workspace(m, n, k)
    arn.set_gemm_splits(splits)
    try:
        plan = check_exact(orc, m, n, k, pre, seed=splits + m, workspace=ws)
    finally:
        arn.set_gemm_splits(0)
    assert "/splits1/" not in plan, plan


@pytest.mark.parametrize("name", ["fp8_gemm_gate_up_13312x16384", "fp8_gemm_down_16384x6656",
                                  "fp8_gemm_qkv_2304x16384", "fp8_gemm_o_16384x2048"])
def test_gemm_exact_full_size(orc, name):
    """The benchmark's shapes in its launch configuration (automatic block
    shape; the QKV shard also with a split-K workspace), both layouts, at
    M = 1 and 64, sampled output columns compared bit for bit."""
    import residual_add_rmsnorm_amd as arn
    import workloads as W

    g = W.GEMMS[name]
    print(f"\n[exact full-size] {name}", flush=True)
    cols = np.unique(np.concatenate([np.linspace(0, g.n - 1, 96).astype(np.int64),
                                     [0, 15, 16, 63, 64, g.n // 2, g.n - 17, g.n - 16,
                                      g.n - 1]]))
    data = exact_data(64, g.n, g.k, seed=len(name))
    for m in (1, 64):
        for pre in (False, True):
            check_exact(orc, m, g.n, g.k, pre, cols=cols, data=data)
    if name == "fp8_gemm_qkv_2304x16384":
        ws = arn.fp8_gemm_workspace(64, g.n, g.k)
        plan = check_exact(orc, 64, g.n, g.k, True, cols=cols, workspace=ws, data=data)
        assert "/splits1/" not in plan, plan
