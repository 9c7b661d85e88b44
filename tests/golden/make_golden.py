"""Write the stored expected/input values under tests/golden/.

Calls only the oracle (and the seeded input generator).  Run from the repo
root:  python tests/golden/make_golden.py

bf16_6656_swiglu_static_scale.json -- the same for the SwiGLU decode
workload (silu(gate) * up, bf16, d 6656).

fp16_16384_static_scale.json -- the per-tensor dequant scale of the decode
workload (fused add + RMSNorm + static e4m3, fp16, hidden 16384).  The
workload fixes the multiplier 448 / (4 * max|y|) over a seed-0 calibration
batch; the library takes the dequant scale s with code = e4m3(y / s), so the
stored value is s = fp32(4 * max|y| / 448), with max|y| taken from the
oracle's unrounded fp64 y over the 256-row seed-0 batch (the decode row
counts 1, 8, 64, 256 are prefixes of that batch).

workload_digests.json -- SHA-256 of the generator's output for the first
rows (up to 256) of every norm, SwiGLU and all-reduce-form workload: x (or
the parts), residual and weight as stored 16-bit patterns, row padding
included.  It pins the draw itself, which the stored static scales above
depend on.  Calls only the generator.
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def static_scale():
    w = workloads.WORKLOADS["fused_add_rmsnorm_fp8_static_fp16_decode_x16384"]
    d = workloads.make(w, rows=256, seed=0)
    r = oracle.oracle().add_rmsnorm(w.dtype, d["x"], d["residual"], d["weight"], w.eps)
    ymax = float(np.max(np.abs(r["y"])))
    s = float(np.float32(4.0 * ymax / 448.0))
    return {
        "workload": w.name,
        "calibration": "seed 0, rows 0..255, oracle fp64 y",
        "max_abs_y": ymax,
        "dequant_scale": s,
        "multiplier": 448.0 / (4.0 * ymax),
    }


def glu_static_scale():
    """The same convention for the SwiGLU decode workload: dequant scale
    s = fp32(4 * max|y| / 448) over its seed-0 256-row calibration batch,
    max|y| from the oracle's fp64 silu(gate) * up."""
    w = workloads.WORKLOADS["silu_and_mul_fp8_static_bf16_decode_x6656"]
    d = workloads.make(w, rows=256, seed=0)
    r = oracle.oracle().silu_and_mul(w.dtype, d["x"], d=w.hidden)
    ymax = float(np.max(np.abs(r["y"])))
    return {
        "workload": w.name,
        "calibration": "seed 0, rows 0..255, oracle fp64 y",
        "max_abs_y": ymax,
        "dequant_scale": float(np.float32(4.0 * ymax / 448.0)),
        "multiplier": 448.0 / (4.0 * ymax),
    }


def digest(d: dict) -> str:
    """SHA-256 over the generator's arrays of one call, in a fixed order."""
    h = hashlib.sha256()
    for key in ("parts", "x", "residual", "weight"):
        v = d.get(key)
        arrays = v if isinstance(v, list) else [v]
        for a in arrays:
            if a is not None:
                h.update(key.encode())
                h.update(str(a.shape).encode())
                h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def workload_digests():
    out = {}
    for name, w in workloads.WORKLOADS.items():
        rows = min(256, w.rows)
        out[name] = {"rows": rows, "sha256": digest(workloads.make(w, rows=rows, seed=0))}
    return {"generator": "workloads.make(w, rows=min(256, w.rows), seed=0)", "workloads": out}


if __name__ == "__main__":
    for name, fn in (("fp16_16384_static_scale.json", static_scale),
                     ("bf16_6656_swiglu_static_scale.json", glu_static_scale),
                     ("workload_digests.json", workload_digests)):
        out = os.path.join(HERE, name)
        with open(out, "w") as f:
            json.dump(fn(), f, indent=1)
            f.write("\n")
        print(open(out).read())
