"""Seeded synthetic inputs for the residual-add + RMSNorm workloads.

This module only draws random numbers and stores them as 16-bit patterns.
It holds none of the operator's arithmetic and imports neither the oracle
nor the HIP library, so both sides can be fed from it.

Generator: numpy's counter-based Philox (Salmon et al., "Parallel random
numbers: as easy as 1, 2, 3", SC'11), keyed by (seed, tensor stream, block of
256 rows).  Keying per row block makes any row range reproducible on its own,
which lets a parity test regenerate sampled rows of a full-size workload
cheaply.  Streams: x = 1, residual = 2, weight = 3, outlier columns = 4;
the partial sums of the all-reduce form use streams 8 + rank.

float32 draws are rounded to bf16 by torch's CPU conversion and to fp16 by
numpy's -- both round to nearest even.

The pages measure only end-to-end serving on model weights, which are not
available here; these draws stand in for activations of the row widths the
workloads name (3840 is the Gemma 4 12B width printed in the MI300X AITER
write-up's untuned-GEMM table).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BLOCK_ROWS = 256
STREAM_X, STREAM_RES, STREAM_W, STREAM_OUTLIER = 1, 2, 3, 4
STREAM_PART0 = 8

# bf16 NaN pattern written into row padding; a kernel that reads it into a
# row's sum of squares turns that row's output into NaN.
PAD_SENTINEL = 0x7FA5


@dataclass(frozen=True)
class Workload:
    name: str
    op: str            # rmsnorm | fused_add_rmsnorm | *_fp8 | silu_and_mul* | sum_add_rmsnorm*
    dtype: str         # bf16 | fp16
    rows: int
    hidden: int
    stride: int
    eps: float
    x_std: float = 1.0
    res_std: float = 1.0
    weight: str = "1+0.1n"          # "1+0.1n" | "u(0.5,1.5)"
    fp8: str | None = None          # None | "static" | "dynamic"
    outliers: int = 0               # columns of x multiplied by outlier_gain
    outlier_gain: float = 50.0
    row_counts: tuple = field(default=())  # decode sweeps: prefixes of `rows`
    nparts: int = 0                 # all-reduce form: ranks whose partial rows are summed

    @property
    def has_residual(self) -> bool:
        return self.op.startswith("fused_add") or self.op.startswith("sum_add")

    @property
    def is_sum(self) -> bool:
        return self.nparts > 0

    @property
    def is_glu(self) -> bool:
        return self.op.startswith("silu_and_mul")

    @property
    def in_width(self) -> int:
        """Columns of x per row: gate | up (2 * hidden) for SwiGLU."""
        return 2 * self.hidden if self.is_glu else self.hidden

    def algorithmic_bytes(self, rows: int | None = None) -> int:
        """Minimum HBM bytes one call must move: 16-bit x read (gate and up
        for SwiGLU), residual read and written, output written (16-bit or
        e4m3), the norm weight once, the static scale read once or the
        dynamic scales written.  The all-reduce form reads every part."""
        r = self.rows if rows is None else rows
        h = self.hidden
        elem = 2
        per_row = self.in_width * elem * max(1, self.nparts)  # x (gate | up; every part)
        if self.has_residual:
            per_row += 2 * h * elem             # residual read + write
        per_row += h * (1 if self.fp8 else elem)  # output
        if self.fp8 == "dynamic":
            per_row += 4
        total = r * per_row
        if not self.is_glu:
            total += h * elem                   # weight once
        if self.fp8 == "static":
            total += 4
        return total


WORKLOADS = {
    w.name: w
    for w in [
        Workload("rmsnorm_bf16_64x4096", "rmsnorm", "bf16", 64, 4096, 4096, 1e-6),
        Workload("fused_add_rmsnorm_bf16_4096x8192", "fused_add_rmsnorm", "bf16",
                 4096, 8192, 8192, 1e-5),
        Workload("fused_add_rmsnorm_fp8_static_fp16_decode_x16384",
                 "fused_add_rmsnorm_fp8", "fp16", 256, 16384, 16384, 1e-5,
                 res_std=2.0, weight="u(0.5,1.5)", fp8="static",
                 row_counts=(1, 8, 64, 256)),
        Workload("fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168",
                 "fused_add_rmsnorm_fp8", "bf16", 32768, 7168, 7168, 1e-6,
                 fp8="dynamic", outliers=8),
        Workload("fused_add_rmsnorm_bf16_65536x3840_stride4096", "fused_add_rmsnorm",
                 "bf16", 65536, 3840, 4096, 1e-6),
        Workload("fused_add_rmsnorm_bf16_65536x2880_stride4096", "fused_add_rmsnorm",
                 "bf16", 65536, 2880, 4096, 1e-6),
        # SwiGLU + e4m3: one GPU's shard of the Llama 3.1 405B MLP (intermediate
        # width 53248 split over the 8 GPUs of one node): d = 6656, rows of
        # gate | up = 13312 columns.
        Workload("silu_and_mul_fp8_dynamic_bf16_32768x6656", "silu_and_mul_fp8", "bf16",
                 32768, 6656, 13312, 0.0, fp8="dynamic"),
        Workload("silu_and_mul_fp8_static_bf16_decode_x6656", "silu_and_mul_fp8", "bf16",
                 256, 6656, 13312, 0.0, fp8="static", row_counts=(1, 8, 64, 256)),
    ]
}

# The all-reduce form, one rank's kernel: 8 tensor-parallel ranks' partial
# sums of a 4096 x 8192 bf16 block output (each partial N(0, 1/8), so the
# total is N(0, 1) like the other workloads' x), then add + norm.
WORKLOADS["sum_add_rmsnorm_bf16_8x4096x8192"] = Workload(
    "sum_add_rmsnorm_bf16_8x4096x8192", "sum_add_rmsnorm", "bf16", 4096, 8192, 8192, 1e-5,
    x_std=float(np.float32(8 ** -0.5)), nparts=8)

# The benchmark's workloads: the five configurations of the operator (the
# strided one at two widths), and the headline among them, the largest
# (65536 x 3840 at row stride 4096: 2.01 GB moved per call).
BENCH_WORKLOADS = (
    "rmsnorm_bf16_64x4096",
    "fused_add_rmsnorm_bf16_4096x8192",
    "fused_add_rmsnorm_fp8_static_fp16_decode_x16384",
    "fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168",
    "fused_add_rmsnorm_bf16_65536x3840_stride4096",
    "fused_add_rmsnorm_bf16_65536x2880_stride4096",
)
HEADLINE = "fused_add_rmsnorm_bf16_65536x3840_stride4096"


def _rng(seed: int, stream: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([seed, stream, block])))


def to_bits(f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the 16-bit type; return the bit patterns."""
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    if dtype == "fp16":
        return f32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(f32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def outlier_columns(w: Workload, seed: int = 0) -> np.ndarray:
    if w.outliers == 0:
        return np.zeros((0,), np.int64)
    cols = _rng(seed, STREAM_OUTLIER, 0).choice(w.hidden, size=w.outliers, replace=False)
    return np.sort(cols.astype(np.int64))


def _normal_rows(seed, stream, row0, row1, hidden, std):
    """float32 N(0, std^2) draws for rows [row0, row1), block-keyed."""
    out = np.empty((row1 - row0, hidden), np.float32)
    b0, b1 = row0 // BLOCK_ROWS, (row1 - 1) // BLOCK_ROWS

    def fill(b):
        blk = _rng(seed, stream, b).standard_normal((BLOCK_ROWS, hidden), dtype=np.float32)
        lo = max(row0, b * BLOCK_ROWS)
        hi = min(row1, (b + 1) * BLOCK_ROWS)
        out[lo - row0:hi - row0] = blk[lo - b * BLOCK_ROWS:hi - b * BLOCK_ROWS]

    # Blocks are independent streams, so they can be drawn in parallel.
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(fill, range(b0, b1 + 1)))
    if std != 1.0:
        out *= np.float32(std)
    return out


def weight_bits(w: Workload, seed: int = 0) -> np.ndarray:
    rng = _rng(seed, STREAM_W, 0)
    if w.weight == "1+0.1n":
        f = 1.0 + 0.1 * rng.standard_normal(w.hidden, dtype=np.float32)
    elif w.weight == "u(0.5,1.5)":
        f = rng.uniform(0.5, 1.5, w.hidden).astype(np.float32)
    else:
        raise ValueError(w.weight)
    return to_bits(f.astype(np.float32), w.dtype)


def padded(bits: np.ndarray, stride: int, fill: int = PAD_SENTINEL) -> np.ndarray:
    rows, width = bits.shape
    if stride == width:
        return bits
    out = np.full((rows, stride), fill, np.uint16)
    out[:, :width] = bits
    return out


def make_rows(w: Workload, row0: int, row1: int, seed: int = 0) -> dict:
    """Inputs for rows [row0, row1) of a workload, rows laid out at the
    workload's stride with padding filled by PAD_SENTINEL.  For SwiGLU, x
    holds gate | up (2 * hidden columns) and there is no weight; the
    all-reduce form has "parts" (one array per rank) instead of x."""
    if w.is_sum:
        out = {"parts": [padded(to_bits(_normal_rows(seed, STREAM_PART0 + g, row0, row1,
                                                     w.hidden, w.x_std), w.dtype), w.stride)
                         for g in range(w.nparts)]}
    else:
        xf = _normal_rows(seed, STREAM_X, row0, row1, w.in_width, w.x_std)
        if w.outliers:
            xf[:, outlier_columns(w, seed)] *= np.float32(w.outlier_gain)
        out = {"x": padded(to_bits(xf, w.dtype), w.stride)}
        del xf
    if w.has_residual:
        rf = _normal_rows(seed, STREAM_RES, row0, row1, w.hidden, w.res_std)
        out["residual"] = padded(to_bits(rf, w.dtype), w.stride)
    out["weight"] = None if w.is_glu else weight_bits(w, seed)
    return out


def make(w: Workload | str, rows: int | None = None, seed: int = 0) -> dict:
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_rows(w, 0, w.rows if rows is None else rows, seed)


# ---------------------------------------------------------------------------
# e4m3 GEMM workloads: the decode-time linear layers of one GPU's share of
# Llama 3.1 405B under 8-way tensor parallelism (hidden 16384, 128 query
# heads and 8 KV heads of width 128, MLP width 53248 -- the model's published
# configuration -- divided by 8 along the parallel dimension).
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class GemmWorkload:
    name: str
    n: int                 # output features (rows of the weight)
    k: int                 # input features
    m_counts: tuple = (1, 8, 16, 32, 64)
    out: str = "bf16"
    a_std: float = 24.0    # activation codes: N(0, a_std^2) cast to e4m3
    b_std: float = 6.0     # weight codes

    def algorithmic_bytes(self, m: int) -> int:
        """Weight codes once, activation codes, 16-bit output, the scales."""
        return self.n * self.k + m * self.k + 2 * m * self.n + 4 * (m + self.n)

    def flops(self, m: int) -> int:
        return 2 * m * self.n * self.k


GEMMS = {
    g.name: g
    for g in [
        GemmWorkload("fp8_gemm_gate_up_13312x16384", 13312, 16384),
        GemmWorkload("fp8_gemm_down_16384x6656", 16384, 6656),
        GemmWorkload("fp8_gemm_qkv_2304x16384", 2304, 16384),
        GemmWorkload("fp8_gemm_o_16384x2048", 16384, 2048),
    ]
}

STREAM_GEMM_A, STREAM_GEMM_B, STREAM_GEMM_SCALE = 5, 6, 7


def e4m3_codes(f32: np.ndarray) -> np.ndarray:
    """float32 values -> OCP e4m3 codes by torch's cast (values clamped to
    the finite range first)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).clamp(-448, 448)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_gemm(g: GemmWorkload, m: int, seed: int = 0) -> dict:
    """Codes and per-row dequant scales for one GEMM call with m rows."""
    a = e4m3_codes(_normal_rows(seed, STREAM_GEMM_A, 0, m, g.k, g.a_std))
    b = e4m3_codes(_normal_rows(seed, STREAM_GEMM_B, 0, g.n, g.k, g.b_std))
    rng = _rng(seed, STREAM_GEMM_SCALE, 0)
    sa = rng.uniform(0.01, 0.1, m).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, g.n).astype(np.float32)
    return {"a": a, "scale_a": sa, "b": b, "scale_b": sb}
