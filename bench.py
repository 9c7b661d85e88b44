"""Benchmark of the fused residual-add + RMSNorm (+ e4m3) HIP path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one call of the operator over one batch of the workload, inputs
already resident in device memory.  With no --workload the run measures
every configuration of the operator and prints ONE JSON line: the headline
is the largest, fused add + RMSNorm, bf16, 65536 rows x 3840 at row stride
4096 (2.01 GB per call), and `config.per_workload` holds the others -- plain
RMSNorm 64 x 4096, fused 4096 x 8192, the decode rows 1/8/64/256 x 16384
with static e4m3 (device time per call from HIP-graph replay and host wall
time per call, beside the launch floor of an empty kernel), dynamic e4m3
32768 x 7168 and the strided 65536 x 2880.  Working sets under four times
the 256 MB Infinity Cache rotate over several buffer sets, so every step
streams from HBM.

Each entry carries the throughput (algorithmic bytes / time), the roofline
fraction of its kernel (average launch duration from HIP events on the
launch stream), the HBM traffic measured by rocprofv3 counters when it was
taken on the current kernel source and launch shape, and the ceiling of a
plain streaming kernel moving the same byte mix.  The headline also carries
the plain CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = ("achieved HBM GB/s (% of MI355X peak) for fused add+RMSNorm(+fp8); "
          "µs/call at decode")
MALL_BYTES = 256 * 1024 * 1024
# Device code of each kernel family: a stored counter reading is used only
# while these files, and the launch shape recorded with it, are unchanged.
_CSRC = "residual_add_rmsnorm_amd/csrc/"
KERNEL_SOURCES = {
    "norm": [_CSRC + "arn_kernels.hip", _CSRC + "arn_device.h", _CSRC + "arn_internal.h"],
    "glu": [_CSRC + "arn_glu.hip", _CSRC + "arn_device.h", _CSRC + "arn_internal.h"],
    "gemm": [_CSRC + "arn_gemm.hip", _CSRC + "arn_device.h", _CSRC + "arn_gemm.h"],
}


def kernel_family(name: str) -> str:
    import workloads

    if name.split("@")[0] in workloads.GEMMS:
        return "gemm"
    return "glu" if workloads.WORKLOADS[name].is_glu else "norm"


def kernel_source_sha(family: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# device-side inputs
# ---------------------------------------------------------------------------

class Batch:
    """Device buffers of one workload, `sets` copies to rotate over."""

    def __init__(self, w, sets: int, rows: int | None = None):
        import torch

        import workloads
        from tests._helpers import dev

        self.w = w
        self.rows = rows or w.rows
        d = workloads.make(w, rows=self.rows)
        H, S = w.hidden, w.stride
        OS = H if w.is_glu else S  # output row stride: dense for SwiGLU
        self.x, self.res, self.out, self.scale = [], [], [], []
        if w.is_sum:
            p0 = [dev(p, w.dtype) for p in d["parts"]]
            x0 = p0[0]
        else:
            x0 = dev(d["x"], w.dtype)
        r0 = dev(d["residual"], w.dtype) if w.has_residual else None
        self.weight = dev(d["weight"], w.dtype) if d["weight"] is not None else None
        for _ in range(sets):
            if w.is_sum:
                self.x.append([p.clone()[:, :w.hidden] for p in p0])
            else:
                self.x.append(x0.clone()[:, :w.in_width])
            self.res.append(r0.clone()[:, :H] if r0 is not None else None)
            if w.fp8:
                o = torch.empty((self.rows, OS), dtype=torch.uint8, device="cuda")
                self.out.append(o.view(torch.float8_e4m3fn)[:, :H])
                if w.fp8 == "dynamic":
                    self.scale.append(torch.empty(self.rows, dtype=torch.float32, device="cuda"))
                else:
                    from tests._helpers import static_scale

                    self.scale.append(torch.tensor([static_scale(w.name)], dtype=torch.float32,
                                                   device="cuda"))
            else:
                self.out.append(torch.empty((self.rows, OS), dtype=x0.dtype, device="cuda")[:, :H])
        del x0, r0
        if w.is_sum:
            del p0
        self.sets = sets

    def call(self, i: int) -> None:
        import residual_add_rmsnorm_amd as arn

        w, k = self.w, i % self.sets
        if w.is_sum:
            kw = {}
            if w.fp8 == "dynamic":
                kw = dict(fp8="dynamic", scales_out=self.scale[k])
            elif w.fp8 == "static":
                kw = dict(fp8="static", scale=self.scale[k])
            arn.sum_add_rmsnorm(self.x[k], self.weight, w.eps, residual=self.res[k],
                                out=self.out[k], **kw)
        elif w.is_glu:
            if w.fp8 == "dynamic":
                arn.silu_and_mul_fp8(self.x[k], dynamic=True, out=self.out[k],
                                     scales_out=self.scale[k])
            elif w.fp8 == "static":
                arn.silu_and_mul_fp8(self.x[k], scale=self.scale[k], out=self.out[k])
            else:
                arn.silu_and_mul(self.x[k], out=self.out[k])
        elif w.fp8:
            kw = dict(dynamic=True, scales_out=self.scale[k]) if w.fp8 == "dynamic" \
                else dict(scale=self.scale[k])
            if w.has_residual:
                arn.fused_add_rmsnorm_fp8(self.x[k], self.res[k], self.weight, w.eps,
                                          out=self.out[k], **kw)
            else:
                arn.rmsnorm_fp8(self.x[k], self.weight, w.eps, out=self.out[k], **kw)
        elif w.has_residual:
            arn.fused_add_rmsnorm(self.x[k], self.res[k], self.weight, w.eps, out=self.out[k])
        else:
            arn.rmsnorm(self.x[k], self.weight, w.eps, out=self.out[k])


def working_set(w, rows) -> int:
    return w.algorithmic_bytes(rows)


def time_steps(batch: Batch, steps: int, warmup: int, min_warm_ms: float = 0.0):
    """(elapsed_ms by HIP events on the launch stream, host wall ms).
    `warmup` untimed calls first; with min_warm_ms, more untimed calls until
    that much time has passed in warm-up."""
    import torch

    for i in range(warmup):
        batch.call(i)
    torch.cuda.synchronize()
    if min_warm_ms > 0:
        t0 = time.perf_counter()
        i = warmup
        while (time.perf_counter() - t0) * 1e3 < min_warm_ms:
            for _ in range(4):
                batch.call(i)
                i += 1
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        batch.call(i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end), wall


def time_graph(batch: Batch, calls: int, replays: int, per_replay: bool = False):
    """Device time per call with host overhead removed: `calls` launches
    captured in one HIP graph, replayed `replays` times.  With per_replay,
    each replay is timed by its own pair of events and (mean, median) of
    the per-call times over the replays is returned."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            batch.call(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            batch.call(i)
    g.replay()
    torch.cuda.synchronize()
    if per_replay:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(replays)]
        for a, b in evs:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        per = [a.elapsed_time(b) * 1e3 / calls for a, b in evs]
        return sum(per) / len(per), statistics.median(per)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (calls * replays)  # us per call


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, single thread, bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(w, target_s: float = 10.0) -> dict:
    """The fp64 C oracle timed on this host on a bounded sample of the same
    workload: single-threaded (the reported value), and once more with the
    sample split into contiguous row ranges over all usable cores (ctypes
    releases the GIL during each oracle call).  Input generation is outside
    the timed region."""
    import concurrent.futures

    import oracle
    import workloads
    from tests._helpers import static_scale

    orc = oracle.oracle()
    mode = {None: oracle.FP8_NONE, "static": oracle.FP8_STATIC,
            "dynamic": oracle.FP8_DYNAMIC}[w.fp8]
    s = static_scale(w.name) if w.fp8 == "static" else 0.0

    def call(d, r0, r1):
        if w.is_sum:
            orc.sum_add_rmsnorm(w.dtype, [p[r0:r1] for p in d["parts"]], d["residual"][r0:r1],
                                d["weight"], w.eps, hidden=w.hidden, fp8_mode=mode,
                                static_scale=s)
        elif w.is_glu:
            orc.silu_and_mul(w.dtype, d["x"][r0:r1], d=w.hidden, fp8_mode=mode, static_scale=s)
        else:
            res = d.get("residual")
            orc.add_rmsnorm(w.dtype, d["x"][r0:r1], None if res is None else res[r0:r1],
                            d["weight"], w.eps, hidden=w.hidden, fp8_mode=mode, static_scale=s)

    def run(rows, threads=1):
        d = workloads.make(w, rows=rows)
        bounds = [rows * i // threads for i in range(threads + 1)]
        t0 = time.perf_counter()
        if threads == 1:
            call(d, 0, rows)
        else:
            with concurrent.futures.ThreadPoolExecutor(threads) as ex:
                list(ex.map(lambda i: call(d, bounds[i], bounds[i + 1]), range(threads)))
        return time.perf_counter() - t0

    probe_rows = min(w.rows, 16)
    t = run(probe_rows)
    rows = int(min(w.rows, max(probe_rows, probe_rows * target_s / max(t, 1e-6))))
    rows = max(1, (rows // 16) * 16) if rows >= 16 else rows
    reps = max(1, min(5, int(target_s / max(t * rows / probe_rows, 1e-6))))
    elapsed = min(run(rows) for _ in range(reps))
    gbs = w.algorithmic_bytes(rows) / elapsed / 1e9
    cores = min(len(os.sched_getaffinity(0)), 16)
    par = min(run(rows, cores) for _ in range(reps))
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {rows} of {w.rows} rows of the same workload, best of {reps} "
                      f"single-threaded fp64 C oracle runs of {elapsed:.1f} s",
            "seconds": round(elapsed, 3),
            "all_cores": {"value": round(w.algorithmic_bytes(rows) / par / 1e9, 4),
                          "cores": cores, "seconds": round(par, 3)}}


def system_info() -> dict:
    """What the run ran on: ROCm and torch versions, the device, and the
    power cap and clocks rocm-smi reports (best effort, never fatal)."""
    import subprocess

    import torch

    info = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    p = torch.cuda.get_device_properties(0)
    info["device"] = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
                      "compute_units": p.multi_processor_count,
                      "memory_GiB": round(p.total_memory / 2**30, 1)}
    try:
        res = subprocess.run(["rocm-smi", "--showpower", "--showmaxpower", "--showclocks",
                              "--json"], capture_output=True, text=True, timeout=20)
        smi = json.loads(res.stdout) if res.returncode == 0 else {}
        card = next(iter(v for k, v in smi.items() if k.startswith("card")), {})
        keep = ("power", "clock", "fclk", "mclk", "sclk", "socclk")
        info["smi"] = {k: v for k, v in card.items() if any(t in k.lower() for t in keep)}
    except (OSError, ValueError, subprocess.TimeoutExpired):
        info["smi"] = None
    return info


# ---------------------------------------------------------------------------
# practical ceilings: plain streaming kernels moving the operator's byte mix
# ---------------------------------------------------------------------------

# (read streams of 16 B, write streams of 16 B, write streams of 8 B) per element
MIXES = {"read": (1, 0, 0), "write": (0, 1, 0), "copy": (1, 1, 0), "2r2w": (2, 2, 0),
         "2r1.5w": (2, 1, 1), "2r0.5w": (2, 0, 1), "9r2w": (9, 2, 0), "9r1.5w": (9, 1, 1)}
PROBE_STREAM_BYTES = 256 * 1024 * 1024


def launch_floor(calls: int = 64, replays: int = 20) -> dict:
    """Time per call of an empty one-block kernel: from HIP-graph replay (as
    the decode rows are timed) and from eager back-to-back launches."""
    import ctypes

    import torch

    from residual_add_rmsnorm_amd import build as _build

    lib = ctypes.CDLL(_build.PROBE_LIB_PATH)
    lib.arn_probe_empty.restype = ctypes.c_int
    lib.arn_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]

    def go():
        st = lib.arn_probe_empty(1, 64, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"arn_probe_empty status {st}")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        go()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            go()
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    t1.synchronize()
    graph_us = t0.elapsed_time(t1) * 1e3 / (calls * replays)
    for _ in range(10):
        go()
    t0.record()
    for _ in range(200):
        go()
    t1.record()
    t1.synchronize()
    eager_us = t0.elapsed_time(t1) * 1e3 / 200
    return {"graph_us_per_call": round(graph_us, 3), "eager_us_per_call": round(eager_us, 3)}


def workload_mix(w):
    """The probe mix with the same read:write byte ratio as the workload."""
    if w.is_sum:
        if w.nparts != 8 or not w.has_residual:
            return None
        return "9r1.5w" if w.fp8 else "9r2w"
    if w.is_glu:
        return "2r0.5w" if w.fp8 else None
    if not w.has_residual:
        return "copy" if not w.fp8 else None
    return "2r1.5w" if w.fp8 else "2r2w"


def mix_ceilings(names, reps: int = 10) -> dict:
    """Best GB/s of the streaming probe (lib/libarn_probe.so) for each mix,
    over block sizes and grids, on 256 MiB streams (64 MiB for the nine-read
    mixes); every call moves far more than the MALL holds."""
    import ctypes

    import torch

    from residual_add_rmsnorm_amd import build as _build

    lib = ctypes.CDLL(_build.PROBE_LIB_PATH)
    lib.arn_probe_stream.restype = ctypes.c_int
    lib.arn_probe_stream.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 4 + [
        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.arn_probe_stream_many.restype = ctypes.c_int
    lib.arn_probe_stream_many.argtypes = [ctypes.c_int] * 3 + [ctypes.c_void_p] * 3 + [
        ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name in names:
        r, w16, w8 = MIXES[name]
        # many-read mixes use shorter streams (every call still moves far
        # more than the MALL holds)
        many = r > 2
        stream_bytes = PROBE_STREAM_BYTES // 4 if many else PROBE_STREAM_BYTES
        n = stream_bytes // 16
        bufs = [torch.empty(stream_bytes, dtype=torch.uint8, device="cuda")
                for _ in range(11 if many else 4)]
        for b in bufs:
            b.fill_(1)
        nbytes = n * (16 * r + 16 * w16 + 8 * w8)
        best = None
        for block in (256, 512, 1024):
            for grid in (256, 512, 1024, 2048, 4096, 8192, n // block):
                srcs = (ctypes.c_void_p * r)(*[b.data_ptr() for b in bufs[:r]])

                def go():
                    if r > 2:
                        st = lib.arn_probe_stream_many(r, w16, w8, srcs, bufs[-2].data_ptr(),
                                                       bufs[-1].data_ptr(), n, grid, block,
                                                       stream)
                    else:
                        st = lib.arn_probe_stream(r, w16, w8, *[b.data_ptr() for b in bufs[:4]],
                                                  n, grid, block, stream)
                    if st != 0:
                        raise RuntimeError(f"arn_probe status {st}")
                for _ in range(3):
                    go()
                t0 = torch.cuda.Event(enable_timing=True)
                t1 = torch.cuda.Event(enable_timing=True)
                t0.record()
                for _ in range(reps):
                    go()
                t1.record()
                t1.synchronize()
                gbs = nbytes * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
                if best is None or gbs > best["GB_per_s"]:
                    best = {"GB_per_s": round(gbs, 1), "block": block, "grid": grid}
        out[name] = best
        log(f"[bench] ceiling {name}: {best}")
        del bufs
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------

def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{name.replace('@', '_')}.json")


def traffic_for(name: str, plan: str):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source and launch shape."""
    path = traffic_file(name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_sha(kernel_family(name)):
        return None
    if t.get("kernel_plan") != plan:
        return None
    return t.get("traffic_bytes_per_launch")


# A freshly placed large workload runs slower for its first ~10-20 ms on
# MI355X (65536 x 2880 at pitch 4096: 270 us/call after 5 warm-up calls,
# 251 us after 50).  The configurations reported beside the headline are
# warmed for at least this long before their timed calls; the headline
# itself takes exactly the requested warm-up steps.
OTHER_MIN_WARM_MS = 30.0


def measure_workload(name: str, steps: int, warmup: int, ceilings: dict | None,
                     min_warm_ms: float = 0.0) -> dict:
    """Time `steps` calls of one workload after `warmup` untimed ones (HIP
    events on the launch stream) and return its entry: per-call time,
    algorithmic GB/s, fraction of the 8 TB/s peak, the launch plan, the
    stored HBM traffic for that plan, and the mix ceiling.  Decode workloads
    add each row count's device time per call from HIP-graph replay and its
    host wall time per call; latency-bound ones (few rows) add their graph
    replay time too."""
    import torch

    import residual_add_rmsnorm_amd as arn
    import workloads

    w = workloads.WORKLOADS[name]
    rows = w.rows
    ws = working_set(w, rows)
    sets = max(1, math.ceil(4 * MALL_BYTES / ws)) if ws < 4 * MALL_BYTES else 1
    sets = min(sets, 64)
    log(f"[bench] {name}: {rows} x {w.hidden} (stride {w.stride}), {sets} buffer set(s)")
    batch = Batch(w, sets)
    elapsed_ms, wall_ms = time_steps(batch, steps, warmup, min_warm_ms)
    plan = arn.last_plan()
    per_call_ms = elapsed_ms / steps
    bytes_step = w.algorithmic_bytes(rows)
    achieved = bytes_step / (per_call_ms * 1e-3) / 1e9
    log(f"[bench] plan {plan}: {per_call_ms * 1e3:.2f} us/call, {achieved:.1f} GB/s "
        f"({100 * achieved / PEAK_HBM_GBS:.1f}% of 8 TB/s)")
    traffic = traffic_for(name, plan)
    entry = {
        "op": w.op, "rows": rows, "hidden": w.hidden, "row_stride": w.stride,
        "io_dtype": w.dtype, "fp8": w.fp8, "eps": w.eps, "buffer_sets": sets,
        **({"nparts": w.nparts} if w.is_sum else {}),
        "bytes_per_call": bytes_step, "kernel_plan": plan,
        "us_per_call": round(per_call_ms * 1e3, 3),
        "GB_per_s": round(achieved, 2),
        "frac_of_hbm_peak": round(achieved / PEAK_HBM_GBS, 4),
        "host_wall_us_per_call": round(wall_ms * 1e3 / steps, 3),
        "traffic_bytes_per_launch": traffic,
        "traffic_over_algorithmic": round(traffic / bytes_step, 5) if traffic else None,
    }
    if min_warm_ms > 0:
        entry["min_warmup_ms"] = min_warm_ms
    mix = workload_mix(w)
    if ceilings is not None and mix:
        if mix not in ceilings:
            ceilings.update(mix_ceilings([mix]))
        c = ceilings[mix]
        entry["mix_ceiling"] = {
            "mix": mix, "GB_per_s": c["GB_per_s"], "frac": round(achieved / c["GB_per_s"], 4),
            "probe": f"plain streaming kernel, block {c['block']}, grid {c['grid']}"}
    if w.row_counts:
        per_rows = {}
        for r in w.row_counts:
            b = Batch(w, 8, rows=r)
            # 30 replays of 64 calls each, timed one by one: the mean, and the
            # median over the 30 (the decode measurement of the MI300X write-up
            # takes the median of 30 iterations)
            dev_us, dev_med = time_graph(b, calls=64, replays=30, per_replay=True)
            e_ms, wall = time_steps(b, 200, 20)
            per_rows[str(r)] = {"device_us_per_call_graph": round(dev_us, 3),
                                "device_us_per_call_graph_median30": round(dev_med, 3),
                                "event_us_per_call": round(e_ms * 1e3 / 200, 3),
                                "host_wall_us_per_call": round(wall * 1e3 / 200, 3),
                                "bytes_per_call": w.algorithmic_bytes(r),
                                "plan": arn.last_plan()}
            log(f"[bench] rows={r}: {per_rows[str(r)]}")
            del b
        entry["decode_us_per_call"] = per_rows
        entry["empty_kernel_launch"] = launch_floor()
    elif rows < 1024:
        b = Batch(w, 8)
        entry["device_us_per_call_graph"] = round(time_graph(b, calls=64, replays=20), 3)
        # eager calls, 200 back to back as for the decode rows, so the final
        # synchronisation does not dominate the host wall time per call
        e_ms, wall = time_steps(b, 200, 20)
        entry["eager_200"] = {"event_us_per_call": round(e_ms * 1e3 / 200, 3),
                              "host_wall_us_per_call": round(wall * 1e3 / 200, 3)}
        entry["empty_kernel_launch"] = launch_floor()
        del b
    del batch
    torch.cuda.empty_cache()
    return entry


def bench_workload(name: str, steps: int, warmup: int, with_cpu: bool,
                   with_ceiling: bool = True, others: tuple = (),
                   head_min_warm_ms: float = 0.0) -> dict:
    """The JSON line of one workload (`name`), optionally with entries for
    `others` under config.per_workload; `head_min_warm_ms` warms `name`
    for at least that long after its `warmup` calls."""
    ceilings = {} if with_ceiling else None
    head = measure_workload(name, steps, warmup, ceilings, head_min_warm_ms)
    per = {}
    for other in others:
        per[other] = measure_workload(other, steps, warmup, ceilings, OTHER_MIN_WARM_MS)
    achieved = head["GB_per_s"]
    config = {"workload": name}
    config.update({k: v for k, v in head.items()
                   if k not in ("GB_per_s", "frac_of_hbm_peak", "traffic_bytes_per_launch",
                                "traffic_over_algorithmic", "mix_ceiling")})
    config["bytes_per_step"] = config.pop("bytes_per_call")
    config["pct_of_hbm_peak"] = round(100 * achieved / PEAK_HBM_GBS, 2)
    if per:
        config["per_workload"] = per
    line = {
        "metric": METRIC,
        "value": achieved,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(head["us_per_call"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": config,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": head["frac_of_hbm_peak"],
            "traffic": head["traffic_bytes_per_launch"],
        },
    }
    if "mix_ceiling" in head:
        line["roofline"]["mix_ceiling"] = head["mix_ceiling"]
    if with_cpu:
        import workloads

        log("[bench] timing the CPU oracle on a bounded sample ...")
        line["cpu_baseline"] = cpu_baseline(workloads.WORKLOADS[name])
        line["system"] = system_info()
    return line


def bench_gemm(name: str, steps: int, warmup: int, only_m: int | None = None,
               only_layout: str | None = None) -> dict:
    """The e4m3 skinny GEMM at each activation row count, with the weight
    pre-shuffled (arn_fp8_gemm_preshuffled, the shuffle done once before the
    timed region), pre-shuffled with a split-K workspace
    (arn_fp8_gemm_preshuffled_ws) and row-major (arn_fp8_gemm): device time
    per call, weight-stream GB/s and TFLOP/s.  Weight copies rotate past the
    Infinity Cache."""
    import torch

    import residual_add_rmsnorm_amd as arn
    import workloads

    g = workloads.GEMMS[name]
    d = workloads.make_gemm(g, max(g.m_counts))
    wbytes = g.n * g.k
    sets = max(1, math.ceil(4 * MALL_BYTES / wbytes))
    log(f"[bench] {name}: n {g.n} k {g.k}, {sets} weight copies")
    b0 = torch.from_numpy(d["b"]).cuda()
    sb = torch.from_numpy(d["scale_b"]).cuda()
    a_all = torch.from_numpy(d["a"]).cuda()
    sa_all = torch.from_numpy(d["scale_a"]).cuda()
    layouts = {"preshuffled": {}, "preshuffled_ws": {}, "rowmajor": {}}
    ws = arn.fp8_gemm_workspace(max(g.m_counts), g.n, g.k)
    for layout in layouts:
        if only_layout and layout != only_layout:
            continue
        if layout.startswith("preshuffled"):
            bs = [arn.fp8_weight_preshuffle(b0) for _ in range(sets)]
        else:
            bs = [b0] + [b0.clone() for _ in range(sets - 1)]
        wsl = ws if layout == "preshuffled_ws" else None
        per_m = layouts[layout]
        for m in g.m_counts:
            if only_m and m != only_m:
                continue
            a, sa = a_all[:m], sa_all[:m]
            out = torch.empty((m, g.n), dtype=torch.bfloat16, device="cuda")

            class _B:
                def call(self, i):
                    arn.fp8_gemm(a, sa, bs[i % sets], sb, out=out, workspace=wsl)

            e_ms, wall = time_steps(_B(), steps, warmup)
            us = e_ms * 1e3 / steps
            per_m[str(m)] = {"us_per_call": round(us, 3),
                             "GB_per_s": round(g.algorithmic_bytes(m) / us / 1e3, 1),
                             "TFLOP_per_s": round(g.flops(m) / us / 1e6, 2),
                             "plan": arn.last_plan()}
            per_m[str(m)]["traffic"] = traffic_for(f"{name}@m{m}_{layout}", per_m[str(m)]["plan"])
            log(f"[bench] {layout} m={m}: {per_m[str(m)]}")
        del bs
        torch.cuda.empty_cache()
    best = max([v for lay in layouts.values() for v in lay.values()],
               key=lambda v: v["GB_per_s"])
    # The roofline entry is the decode case: one activation row, pre-shuffled
    # weight (the configuration the committed counters cover); the best line
    # over every row count and layout is reported beside it.
    head = layouts["preshuffled"].get("1", best)
    return {"workload": name, "n": g.n, "k": g.k, "weight_copies": sets,
            "empty_kernel_launch": launch_floor(),
            "per_m": layouts["preshuffled"], "per_m_splitk": layouts["preshuffled_ws"],
            "per_m_rowmajor": layouts["rowmajor"],
            "roofline": {"bound": "hbm", "achieved": head["GB_per_s"], "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(head["GB_per_s"] / PEAK_HBM_GBS, 4),
                         "traffic": head["traffic"], "plan": head["plan"],
                         "best_GB_per_s": best["GB_per_s"], "best_plan": best["plan"]}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=None,
                    help="one workload name (one line), 'all' (one line each), 'gemms'; "
                         "default: the headline with every configuration in one line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-probe ceiling of the workload's byte mix")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the streaming-probe ceilings of every mix")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run plain device copies of a known size (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                         "`bench.py --calibrate-copy` into profiles/traffic_<workload>.json")
    ap.add_argument("--pmc-command", default="", help="command line recorded with the summary")
    ap.add_argument("--row-probe", action="store_true",
                    help="only time the row-ordered 2R2W probe in every access order beside "
                         "the fused kernel")
    ap.add_argument("--launch-traffic", action="store_true",
                    help="only run the plain norm at a few row counts with and without a weight "
                         "(run it under rocprofv3 --pmc to separate fixed bytes per launch)")
    ap.add_argument("--summarize-launch-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="fit the two counter runs of --launch-traffic into "
                         "profiles/launch_traffic_rmsnorm_bf16_x4096.json")
    ap.add_argument("--pmc-bench-output", default=None,
                    help="the JSON line the profiled bench run printed (its kernel plan is "
                         "recorded with the summary)")
    ap.add_argument("--gemm-m", type=int, default=None,
                    help="GEMM workloads: time only this activation row count")
    ap.add_argument("--gemm-layout", choices=("preshuffled", "preshuffled_ws", "rowmajor"),
                    default=None,
                    help="GEMM workloads: time only this weight layout")
    args = ap.parse_args()

    if args.summarize_pmc:
        import workloads

        summarize_pmc(args.workload or workloads.HEADLINE, *args.summarize_pmc,
                      command=args.pmc_command, bench_output=args.pmc_bench_output,
                      gemm_m=args.gemm_m, gemm_layout=args.gemm_layout)
        return 0

    if args.summarize_launch_traffic:
        summarize_launch_traffic(*args.summarize_launch_traffic, command=args.pmc_command)
        return 0

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the operator is row-independent: rows shard across GPUs with no exchange, "
              "so per-GPU throughput is the single-GPU figure)", file=sys.stderr)
        return 2

    import torch

    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    from residual_add_rmsnorm_amd import _lib

    _lib.load()  # fails loudly if the HIP library is missing

    if args.launch_traffic:
        launch_traffic_sweep()
        return 0

    if args.row_probe:
        print(json.dumps({"row_order_probe": row_order_probe()}), flush=True)
        return 0

    if args.ceilings:
        print(json.dumps({"ceilings_GB_per_s": mix_ceilings(list(MIXES)),
                          "stream_bytes": {"two-stream mixes": PROBE_STREAM_BYTES,
                                           "nine-stream mixes": PROBE_STREAM_BYTES // 4}}),
              flush=True)
        return 0

    if args.workload in workloads.GEMMS or args.workload == "gemms":
        gnames = list(workloads.GEMMS) if args.workload == "gemms" else [args.workload]
        for n in gnames:
            print(json.dumps(bench_gemm(n, min(args.steps, 200), min(args.warmup, 20),
                                        args.gemm_m, args.gemm_layout)), flush=True)
        if args.calibrate_copy:
            copy_calibration()
        return 0
    if args.workload is None:
        # the default run: the headline with every other configuration in
        # config.per_workload, one JSON line
        others = tuple(n for n in workloads.BENCH_WORKLOADS if n != workloads.HEADLINE)
        line = bench_workload(workloads.HEADLINE, args.steps, args.warmup,
                              with_cpu=not args.no_cpu_baseline,
                              with_ceiling=not args.no_ceiling, others=others)
        print(json.dumps(line), flush=True)
        if args.calibrate_copy:
            copy_calibration()
        return 0
    names = list(workloads.WORKLOADS) if args.workload == "all" else [args.workload]
    # one line per workload: each is warmed like the default run's
    # non-headline configurations (a single named workload takes exactly the
    # requested warm-up calls, as the profiled commands assume)
    warm_ms = OTHER_MIN_WARM_MS if args.workload == "all" else 0.0
    for n in names:
        line = bench_workload(n, args.steps, args.warmup,
                              with_cpu=not args.no_cpu_baseline and n == names[0],
                              with_ceiling=not args.no_ceiling, head_min_warm_ms=warm_ms)
        print(json.dumps(line), flush=True)
    if args.calibrate_copy:
        copy_calibration()
    return 0


COPY_BYTES = 256 * 1024 * 1024
COPY_REPS = 10


def _pmc_rows(path: str, counter: str):
    import csv

    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def summarize_pmc(name: str, fetch_csv: str, write_csv: str, command: str = "",
                  bench_output: str | None = None, gemm_m: int | None = None,
                  gemm_layout: str | None = None) -> dict:
    """HBM traffic of the operator's kernel per launch, from FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch), each scaled by what the same counter
    reads for the plain device copies of COPY_BYTES that close the run.
    For a GEMM workload the run timed one row count and layout (the weight
    shuffle dispatched before it is left out)."""
    import workloads

    if name in workloads.GEMMS:
        if not gemm_m or not gemm_layout:
            raise SystemExit("a GEMM summary needs --gemm-m and --gemm-layout")
        key = f"{name}@m{gemm_m}_{gemm_layout}"
        alg = workloads.GEMMS[name].algorithmic_bytes(gemm_m)
    else:
        key = name
        alg = workloads.WORKLOADS[name].algorithmic_bytes()
    plan = None
    if bench_output:
        with open(bench_output) as f:
            line = json.loads(f.readline())
        if "per_m" in line:
            lay = {"preshuffled": line["per_m"], "preshuffled_ws": line["per_m_splitk"],
                   "rowmajor": line["per_m_rowmajor"]}[gemm_layout]
            plan = lay[str(gemm_m)]["plan"]
        else:
            plan = line["config"]["kernel_plan"]
    out = {"workload": key, "kernel_source_sha": kernel_source_sha(kernel_family(key)),
           "kernel_plan": plan, "algorithmic_bytes_per_launch": alg, "command": command}
    want_items = plan_work_items(plan) if plan else None
    for counter, path, kind in (("FETCH_SIZE", fetch_csv, "read"), ("WRITE_SIZE", write_csv, "write")):
        rows = _pmc_rows(path, counter)
        kern = [float(r["Counter_Value"]) for r in rows
                if r["Kernel_Name"].startswith("void arn::")
                and "preshuffle_kernel" not in r["Kernel_Name"]
                and (want_items is None or "Grid_Size" not in r
                     or int(r["Grid_Size"]) == want_items)]
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"]][-COPY_REPS:]
        kib = sum(kern) / len(kern)
        copy_kib = sum(copies) / len(copies)
        factor = COPY_BYTES / (copy_kib * 1024.0)
        out[f"{kind}_counter_kib_per_launch"] = round(kib, 3)
        out[f"{kind}_copy_counter_kib"] = round(copy_kib, 3)
        out[f"{kind}_scale_factor"] = round(factor, 6)
        out[f"{kind}_bytes_per_launch"] = int(round(kib * 1024.0 * factor))
        out[f"{kind}_dispatches"] = len(kern)
    out["traffic_bytes_per_launch"] = out["read_bytes_per_launch"] + out["write_bytes_per_launch"]
    out["traffic_over_algorithmic"] = round(out["traffic_bytes_per_launch"] / alg, 5)
    with open(traffic_file(key), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(json.dumps(out, indent=1))
    return out


def plan_work_items(plan: str):
    """Work-items of one launch of a norm-family plan string
    (".../wpr8/nv2/rpb1/grid4096": 4096 blocks of 64 * 8 * 1 threads), the
    Grid_Size rocprofv3 records per dispatch; None for other plans.  A run
    that also launches other row counts (the decode sweep) is summarised
    over the dispatches of the recorded plan only."""
    import re

    m = re.search(r"/wpr(\d+)/nv\d+/rpb(\d+)/grid(\d+)$", plan)
    if not m:
        return None
    wpr, rpb, grid = (int(g) for g in m.groups())
    return grid * 64 * wpr * rpb


# Access order of the fused norm's row traffic: the row-ordered 2R2W probe
# (arn_probe_rows) in every order and rows per block, next to the fused
# kernel itself and the grid-stride 2R2W probe, at the strided 3840-wide row
# shape (65536 rows, pitch 4096) and at a 8192-wide row (32768 rows).
ROW_PROBE_SHAPES = (("65536x3840_stride4096", 65536, 3840, 4096),
                    ("32768x8192", 32768, 8192, 8192))


def row_order_probe(reps: int = 20) -> dict:
    import ctypes

    import torch

    import residual_add_rmsnorm_amd as arn
    from residual_add_rmsnorm_amd import build as _build

    lib = ctypes.CDLL(_build.PROBE_LIB_PATH)
    f = lib.arn_probe_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 3 + [
        ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream

    def timed(go):
        for _ in range(3):
            go()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            go()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    out = {}
    for name, rows, hidden, stride in ROW_PROBE_SHAPES:
        n = rows * stride
        x = torch.randn(n, device="cuda").to(torch.bfloat16)
        r = torch.randn(n, device="cuda").to(torch.bfloat16)
        o = torch.empty(n, dtype=torch.bfloat16, device="cuda")
        nbytes = rows * hidden * 2 * 4
        res = {}
        xv, rv, ov = (t.view(rows, stride)[:, :hidden] for t in (x, r, o))
        w = torch.ones(hidden, dtype=torch.bfloat16, device="cuda")
        # the kernel first and last, so a drift over the run shows
        for tag in ("fused_kernel_first",):
            us = timed(lambda: arn.fused_add_rmsnorm(xv, rv, w, 1e-6, out=ov))
            res[tag] = {"us": round(us, 2), "GB_per_s": round((nbytes + 2 * hidden) / us / 1e3, 1),
                        "plan": arn.last_plan()}
        for g in (1, 2, 4):
            for mode in (0, 1, 2, 3):
                if g == 1 and mode:
                    continue

                def go():
                    rc = f(mode, g, x.data_ptr(), r.data_ptr(), o.data_ptr(), rows, hidden * 2,
                           stride * 2, st)
                    if rc != 0:
                        raise RuntimeError(f"arn_probe_rows status {rc}")
                us = timed(go)
                res[f"rows_per_block{g}_mode{mode}"] = {"us": round(us, 2),
                                                        "GB_per_s": round(nbytes / us / 1e3, 1)}
        us = timed(lambda: arn.fused_add_rmsnorm(xv, rv, w, 1e-6, out=ov))
        res["fused_kernel_last"] = {"us": round(us, 2),
                                    "GB_per_s": round((nbytes + 2 * hidden) / us / 1e3, 1),
                                    "plan": arn.last_plan()}
        log(f"[bench] row probe {name}: {res}")
        out[name] = res
        del x, r, o, xv, rv, ov
        torch.cuda.empty_cache()
    out["grid_stride_2r2w"] = mix_ceilings(["2r2w"])["2r2w"]
    return out


# Fixed traffic per launch: the plain norm 4096 wide (the rmsnorm workload's
# width) at two row counts with the weight and two without, 20 launches each
# over 8 rotating buffer sets, then the calibration copies.  Under two
# rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) this separates the bytes per
# row, the weight's bytes per launch and a fixed remainder per launch.
SWEEP_HIDDEN = 4096
SWEEP_CASES = ((64, True), (65, False), (256, True), (257, False))
SWEEP_LAUNCHES = 20


def launch_traffic_sweep() -> None:
    import torch

    import residual_add_rmsnorm_amd as arn

    rmax = max(r for r, _ in SWEEP_CASES)
    xs = [torch.randn(rmax, SWEEP_HIDDEN, device="cuda").to(torch.bfloat16) for _ in range(8)]
    outs = [torch.empty_like(xs[0]) for _ in range(8)]
    w = torch.full((SWEEP_HIDDEN,), 1.5, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    for rows, with_w in SWEEP_CASES:
        for i in range(SWEEP_LAUNCHES):
            arn.rmsnorm(xs[i % 8][:rows], w if with_w else None, 1e-6, out=outs[i % 8][:rows])
        torch.cuda.synchronize()
        log(f"[bench] launch-traffic sweep: {rows} rows, weight {with_w}, plan {arn.last_plan()}")
    copy_calibration()


def summarize_launch_traffic(fetch_csv: str, write_csv: str, command: str = "") -> dict:
    """Per case of SWEEP_CASES (told apart by their grids: one block of 512
    threads per row), the mean FETCH_SIZE and WRITE_SIZE bytes per launch
    (scaled by the calibration copies), and the fit: bytes per row from the
    two weightless cases, the fixed remainder per launch, and the weight's
    bytes per launch."""
    out = {"hidden": SWEEP_HIDDEN, "cases": [], "command": command}
    per = {}
    for counter, path, kind in (("FETCH_SIZE", fetch_csv, "read"), ("WRITE_SIZE", write_csv, "write")):
        rows = _pmc_rows(path, counter)
        copies = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]][-COPY_REPS:]
        factor = COPY_BYTES / (sum(copies) / len(copies) * 1024.0)
        for nrows, with_w in SWEEP_CASES:
            vals = [float(r["Counter_Value"]) for r in rows
                    if r["Kernel_Name"].startswith("void arn::") and int(r["Grid_Size"]) == nrows * 512]
            per[(nrows, with_w, kind)] = sum(vals) / len(vals) * 1024.0 * factor
    for nrows, with_w in SWEEP_CASES:
        out["cases"].append({"rows": nrows, "weight": with_w,
                             "read_bytes_per_launch": round(per[(nrows, with_w, "read")]),
                             "write_bytes_per_launch": round(per[(nrows, with_w, "write")])})
    (r0, _), (r1, _) = [c for c in SWEEP_CASES if not c[1]]
    row_bytes = (per[(r1, False, "read")] - per[(r0, False, "read")]) / (r1 - r0)
    fixed = per[(r0, False, "read")] - r0 * row_bytes
    weight = [per[(r, True, "read")] - fixed - r * row_bytes for r, w in SWEEP_CASES if w]
    out["fit"] = {"read_bytes_per_row": round(row_bytes, 1),
                  "read_fixed_bytes_per_launch": round(fixed),
                  "read_weight_bytes_per_launch": [round(v) for v in weight],
                  "weight_bytes": SWEEP_HIDDEN * 2}
    path = os.path.join(ROOT, "profiles", "launch_traffic_rmsnorm_bf16_x4096.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(json.dumps(out, indent=1))
    return out


def copy_calibration(reps: int = 10) -> None:
    """Plain device-to-device copies of COPY_BYTES (read COPY_BYTES, write
    COPY_BYTES): the reference that scales the HBM byte counters."""
    import torch

    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = [torch.empty_like(src) for _ in range(2)]
    for i in range(reps):
        dst[i % 2].copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {COPY_BYTES} bytes")


if __name__ == "__main__":
    sys.exit(main())
