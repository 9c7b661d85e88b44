"""The norm's launch plan (access width and tile) through arn_norm_plan,
without a GPU: the plans the committed HBM-counter summaries were taken
under, the decode-batch tile bands on both sides of each boundary and at
another CU count, and properties every accepted plan has."""
import glob
import json
import os
import re

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import residual_add_rmsnorm_amd as arn
import workloads as W
from residual_add_rmsnorm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PLAN = re.compile(r"^(sum_)?(\w+)/(bf16|fp16)/vec(\d+)/wpr(\d+)/nv(\d+)/rpb(\d+)/grid(\d+)$")


def _norm_traffic_files():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))):
        with open(path) as f:
            t = json.load(f)
        w = W.WORKLOADS.get(t.get("workload"))
        if w is not None and w.op in ("rmsnorm", "fused_add_rmsnorm", "fused_add_rmsnorm_fp8",
                                      "rmsnorm_fp8"):
            out.append((t["workload"], t["kernel_plan"]))
    return out


@pytest.mark.parametrize("name,plan", _norm_traffic_files())
def test_profiled_plans_are_the_ones_chosen(name, plan):
    """Each committed counter summary names the plan it was taken under;
    on a 256-CU device the library still chooses exactly that plan."""
    w = W.WORKLOADS[name]
    got = arn.norm_plan(w.dtype, w.rows, w.hidden, fused=w.has_residual, fp8=w.fp8,
                        stride=w.stride, weight=True)
    assert got == plan


# (dtype, rows per CU, extra rows, hidden, fp8) -> tile, fused kinds with
# 128-bit accesses; rows = int(rows per CU * CUs) + extra rows
BANDS = [
    ("bf16", 0.0, 1, 8192, None, "wpr8/nv2"),       # bf16 at <= 1/2 row per CU: eight waves
    ("fp16", 0.0, 1, 8192, None, "wpr4/nv4"),       # fp16 there: four waves
    ("fp16", 0.5, 0, 5120, "static", "wpr4/nv3"),
    ("bf16", 0.5, 0, 7168, "dynamic", "wpr8/nv2"),
    ("bf16", 0.5, 1, 7168, "dynamic", "wpr4/nv4"),  # just past half a row per CU
    ("bf16", 1.0, 0, 8192, None, "wpr4/nv4"),
    ("bf16", 1.25, 0, 8192, "static", "wpr4/nv4"),
    ("bf16", 1.25, 1, 8192, "static", "wpr2/nv8"),  # just past 1.25
    ("fp16", 1.25, 1, 5120, None, "wpr4/nv3"),      # 640 vectors: four waves stay
    ("fp16", 2.0, 0, 7168, None, "wpr2/nv8"),
    ("fp16", 2.0, 1, 7168, None, "wpr8/nv2"),       # past two rows per CU
    ("bf16", 1.0, 0, 4096, None, "wpr8/nv1"),       # 512 vectors: outside the bands
    ("bf16", 1.0, 0, 8200, None, "wpr8/nv4"),       # 1025 vectors: outside
]


@pytest.mark.parametrize("cus", [256, 304])
@pytest.mark.parametrize("dtype,per_cu,extra,hidden,fp8,tile", BANDS)
def test_decode_batch_bands(dtype, per_cu, extra, hidden, fp8, tile, cus):
    """The fused decode-batch tile bands, on both sides of each boundary,
    scale with the CU count."""
    rows = int(per_cu * cus) + extra
    got = arn.norm_plan(dtype, rows, hidden, fused=True, fp8=fp8, compute_units=cus)
    assert f"/vec8/{tile}/" in got, got


def test_bands_are_fused_only_and_need_full_width_access():
    # plain kinds at one row per CU keep eight waves
    assert "/wpr8/nv2/" in arn.norm_plan("fp16", 256, 8192)
    # 8-byte aligned bases allow only 4-element accesses: general rule
    got = arn.norm_plan("fp16", 256, 8192, fused=True, align=8)
    assert "/vec4/" in got and "/wpr16/" in got, got


def test_many_rows_and_decode_rules():
    # fused kinds with many rows: eight waves, two vectors
    assert "/vec8/wpr8/nv2/rpb1/" in arn.norm_plan("bf16", 4096, 8192, fused=True)
    # plain kinds with many rows: compact tiles
    assert "/vec8/wpr4/nv4/rpb1/" in arn.norm_plan("bf16", 1030, 7168)
    assert "/vec8/wpr1/nv2/rpb4/" in arn.norm_plan("bf16", 1030, 1024, fp8="dynamic")
    # the decode benchmark's rows: eight waves, four vectors
    for r in (1, 8, 64, 256):
        assert arn.norm_plan("fp16", r, 16384, fused=True, fp8="static") == \
            f"fused_add_fp8s/fp16/vec8/wpr8/nv4/rpb1/grid{r}"


def test_forced_tile_applies_to_the_query():
    arn.set_tile(16, 2)
    try:
        assert "/wpr16/nv2/" in arn.norm_plan("bf16", 4096, 8192, fused=True)
        with pytest.raises(_lib.ArnError):  # 16 x 64 x 2 x 8 < 32768
            arn.norm_plan("bf16", 4, 32768, fused=True)
    finally:
        arn.set_tile(0, 0)
    assert "/wpr8/nv2/" in arn.norm_plan("bf16", 4096, 8192, fused=True)


def test_query_refusals_match_the_call():
    with pytest.raises(_lib.ArnError) as e:
        arn.norm_plan("bf16", 4, 65537)  # 2-byte rows above 16384 elements
    assert e.value.status == _lib.EUNSUPPORTED
    with pytest.raises(_lib.ArnError) as e:
        arn.norm_plan("bf16", 4, 64, stride=32)  # stride below hidden
    assert e.value.status == _lib.EINVAL
    with pytest.raises(_lib.ArnError) as e:
        arn.norm_plan("bf16", 4, 64, compute_units=0)
    assert e.value.status == _lib.EINVAL
    assert arn.norm_plan("bf16", 0, 64) == ""


@settings(max_examples=400, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.too_slow])
@given(dtype=st.sampled_from(["bf16", "fp16"]), rows=st.integers(1, 1 << 24),
       hidden=st.integers(1, 65536), pad=st.integers(0, 64), fused=st.booleans(),
       fp8=st.sampled_from([None, "static", "dynamic"]), align=st.sampled_from([2, 4, 8, 16]),
       cus=st.sampled_from([32, 80, 256, 304]))
def test_every_accepted_plan_covers_its_rows(dtype, rows, hidden, pad, fused, fp8, align, cus):
    """Any plan the query accepts: the widest access the row length, the
    strides and the bases allow; a tile whose lanes cover the row; the last
    launch's grid holds the rows past the previous launches (2^22 blocks
    each).  A refusal is only ever for rows too long for every tile."""
    stride = hidden + pad
    # every base the query passes is aligned to exactly `align` bytes; a
    # 16-bit access of `vec` elements needs 2 * vec
    widest = 8
    while widest > 1 and not (hidden % widest == 0 and stride % widest == 0 and
                              align % (2 * widest) == 0):
        widest //= 2
    longest = {1: 16384, 2: 32768, 4: 65536, 8: 65536}[widest]  # served row lengths (arn.h)
    try:
        got = arn.norm_plan(dtype, rows, hidden, fused=fused, fp8=fp8, stride=stride, align=align,
                            compute_units=cus)
    except _lib.ArnError as e:
        assert e.status == _lib.EUNSUPPORTED and hidden > longest, (e.status, hidden, widest)
        return
    assert hidden <= longest
    m = PLAN.match(got)
    assert m, got
    vec, wpr, nv, rpb, grid = (int(m.group(i)) for i in range(4, 9))
    assert vec == widest, (got, align)
    assert 64 * wpr * nv * vec >= hidden
    per_launch = (1 << 22) * rpb
    last = rows - (rows - 1) // per_launch * per_launch
    assert grid == -(-last // rpb)
