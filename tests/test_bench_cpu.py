"""Host logic of bench.py, without a GPU: the algorithmic byte counts that
every GB/s figure divides by (against sums written out by hand from the
tensor sizes), the scaling of rocprofv3's FETCH_SIZE / WRITE_SIZE readings
by the calibration copies, the rule that a stored traffic reading is used
only for the kernel source and launch shape it was taken on, the byte mix
each workload is compared with, and the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MiB = 1 << 20


def test_algorithmic_bytes_by_hand():
    # fused add + norm, bf16 4096 x 8192: x read, residual read + written,
    # out written (64 MiB each), weight 16 KiB once
    assert W.WORKLOADS["fused_add_rmsnorm_bf16_4096x8192"].algorithmic_bytes() == \
        4 * 64 * MiB + 8192 * 2
    # dynamic e4m3, 32768 x 7168: 16-bit x, residual r + w, 1-byte codes,
    # one fp32 scale per row, weight once
    r, h = 32768, 7168
    assert W.WORKLOADS["fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168"].algorithmic_bytes() == \
        r * h * (2 + 4 + 1) + 4 * r + 2 * h
    # strided rows count only the hidden columns, never the padding
    r, h = 65536, 3840
    assert W.WORKLOADS["fused_add_rmsnorm_bf16_65536x3840_stride4096"].algorithmic_bytes() == \
        r * h * 8 + 2 * h
    # plain norm: x read, out written
    assert W.WORKLOADS["rmsnorm_bf16_64x4096"].algorithmic_bytes() == 64 * 4096 * 4 + 4096 * 2
    # SwiGLU + dynamic e4m3: gate and up read, codes and scales written
    r, d = 32768, 6656
    assert W.WORKLOADS["silu_and_mul_fp8_dynamic_bf16_32768x6656"].algorithmic_bytes() == \
        r * (4 * d + d + 4)
    # all-reduce form over 8 parts: every part read, residual r + w, out, weight
    r, h = 4096, 8192
    assert W.WORKLOADS["sum_add_rmsnorm_bf16_8x4096x8192"].algorithmic_bytes() == \
        r * h * 2 * (8 + 2 + 1) + 2 * h
    # GEMM: weight codes once, activation codes, 16-bit output, both scales
    g = W.GEMMS["fp8_gemm_gate_up_13312x16384"]
    assert g.algorithmic_bytes(1) == 13312 * 16384 + 16384 + 2 * 13312 + 4 * (1 + 13312)
    assert g.flops(64) == 2 * 64 * 13312 * 16384


def test_workload_mix():
    mix = {name: bench.workload_mix(w) for name, w in W.WORKLOADS.items()}
    assert mix["fused_add_rmsnorm_bf16_4096x8192"] == "2r2w"
    assert mix["fused_add_rmsnorm_fp8_dynamic_bf16_32768x7168"] == "2r1.5w"
    assert mix["rmsnorm_bf16_64x4096"] == "copy"
    assert mix["silu_and_mul_fp8_dynamic_bf16_32768x6656"] == "2r0.5w"
    assert mix["sum_add_rmsnorm_bf16_8x4096x8192"] == "9r2w"
    for m in mix.values():
        assert m is None or m in bench.MIXES


def _counter_csv(path, counter, kernel_kib, copy_kib, copies=bench.COPY_REPS, grid=None,
                 other_grid_kib=()):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Grid_Size", "Kernel_Name",
                                          "Counter_Name", "Counter_Value"])
        w.writeheader()
        i = 0
        for v in kernel_kib:
            i += 1
            w.writerow({"Dispatch_Id": i, "Grid_Size": grid or 1,
                        "Kernel_Name": "void arn::row_kernel<0>(arn::Args)",
                        "Counter_Name": counter, "Counter_Value": v})
        for v in other_grid_kib:   # the same kernel at another row count
            i += 1
            w.writerow({"Dispatch_Id": i, "Grid_Size": 512,
                        "Kernel_Name": "void arn::row_kernel<0>(arn::Args)",
                        "Counter_Name": counter, "Counter_Value": v})
        i += 1
        w.writerow({"Dispatch_Id": i, "Grid_Size": 64, "Kernel_Name": "void some_other_kernel()",
                    "Counter_Name": counter, "Counter_Value": 1e9})
        for _ in range(copies):
            i += 1
            w.writerow({"Dispatch_Id": i, "Grid_Size": 1 << 20,
                        "Kernel_Name": "__amd_rocclr_copyBuffer",
                        "Counter_Name": counter, "Counter_Value": copy_kib})


def test_summarize_pmc_scaling(tmp_path, monkeypatch):
    """Each counter is scaled by COPY_BYTES over what it read for the copies;
    kernels other than the operator's are left out."""
    name = "fused_add_rmsnorm_bf16_4096x8192"
    alg = W.WORKLOADS[name].algorithmic_bytes()
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the fetch counter reads half of the copy's bytes (as on the GPU host),
    # the write counter all of them
    _counter_csv(fetch, "FETCH_SIZE", [alg / 2 / 1024 / 2] * 3, copy_kib / 2)
    _counter_csv(write, "WRITE_SIZE", [alg / 2 / 1024] * 3, copy_kib)
    out_json = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda key: str(out_json))
    out = bench.summarize_pmc(name, str(fetch), str(write), command="test")
    assert out["read_scale_factor"] == pytest.approx(2.0)
    assert out["write_scale_factor"] == pytest.approx(1.0)
    assert out["read_dispatches"] == 3
    assert out["traffic_bytes_per_launch"] == pytest.approx(alg, abs=2)
    assert out["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert json.loads(out_json.read_text())["kernel_source_sha"] == \
        bench.kernel_source_sha("norm")


def test_traffic_used_only_for_its_source_and_plan(tmp_path, monkeypatch):
    name = "fused_add_rmsnorm_bf16_4096x8192"
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "traffic_file", lambda key: str(path))
    assert bench.traffic_for(name, "p") is None  # no reading stored
    rec = {"kernel_source_sha": bench.kernel_source_sha("norm"), "kernel_plan": "p",
           "traffic_bytes_per_launch": 123}
    path.write_text(json.dumps(rec))
    assert bench.traffic_for(name, "p") == 123
    assert bench.traffic_for(name, "other plan") is None
    path.write_text(json.dumps(dict(rec, kernel_source_sha="0" * 16)))
    assert bench.traffic_for(name, "p") is None


def test_kernel_families():
    assert bench.kernel_family("fused_add_rmsnorm_bf16_4096x8192") == "norm"
    assert bench.kernel_family("sum_add_rmsnorm_bf16_8x4096x8192") == "norm"
    assert bench.kernel_family("silu_and_mul_fp8_dynamic_bf16_32768x6656") == "glu"
    assert bench.kernel_family("fp8_gemm_qkv_2304x16384@m16_preshuffled_ws") == "gemm"
    for srcs in bench.KERNEL_SOURCES.values():
        for p in srcs:
            assert os.path.exists(os.path.join(ROOT, p)), p


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stdout + res.stderr


def test_default_run_covers_every_configuration_with_the_largest_as_headline():
    """The default bench line measures all five configurations (the strided
    one at both widths); its headline is the one that moves the most bytes."""
    names = W.BENCH_WORKLOADS
    assert len(names) == len(set(names)) == 6
    assert W.HEADLINE in names
    assert W.HEADLINE == max(names, key=lambda n: W.WORKLOADS[n].algorithmic_bytes())
    assert W.WORKLOADS[W.HEADLINE].algorithmic_bytes() == 65536 * 3840 * 8 + 3840 * 2
    ops = {W.WORKLOADS[n].op for n in names}
    assert ops == {"rmsnorm", "fused_add_rmsnorm", "fused_add_rmsnorm_fp8"}
    decode = [n for n in names if W.WORKLOADS[n].row_counts]
    assert decode == ["fused_add_rmsnorm_fp8_static_fp16_decode_x16384"]
    assert W.WORKLOADS[decode[0]].row_counts == (1, 8, 64, 256)


def test_summarize_pmc_keeps_the_recorded_plans_dispatches(tmp_path, monkeypatch):
    """A run that also launches other row counts (the decode sweep) is
    summarised over the dispatches whose grid matches the recorded plan."""
    name = "fused_add_rmsnorm_fp8_static_fp16_decode_x16384"
    plan = "fused_add_fp8s/fp16/vec8/wpr8/nv4/rpb1/grid256"
    assert bench.plan_work_items(plan) == 256 * 512
    assert bench.plan_work_items("fp8_gemm/bf16/mt1/nt1/waves8/splits1/grid144") is None
    alg = W.WORKLOADS[name].algorithmic_bytes()
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, "FETCH_SIZE", [alg * 4 / 7 / 1024] * 3, copy_kib, grid=256 * 512,
                 other_grid_kib=[1.0, 2.0])
    _counter_csv(write, "WRITE_SIZE", [alg * 3 / 7 / 1024] * 3, copy_kib, grid=256 * 512,
                 other_grid_kib=[3.0])
    line = tmp_path / "line.json"
    line.write_text(json.dumps({"config": {"kernel_plan": plan}}) + "\n")
    monkeypatch.setattr(bench, "traffic_file", lambda key: str(tmp_path / "t.json"))
    out = bench.summarize_pmc(name, str(fetch), str(write), bench_output=str(line))
    assert out["read_dispatches"] == 3 and out["write_dispatches"] == 3
    assert out["traffic_over_algorithmic"] == pytest.approx(1.0, abs=1e-6)


def test_launch_traffic_fit(tmp_path, monkeypatch):
    """The sweep's fit recovers bytes per row, a fixed remainder per launch
    and the weight's bytes from synthetic counter files built with them."""
    per_row, fixed, weight = 8192, 48000, 8 * 8192
    rows = []
    i = 0
    for nrows, with_w in bench.SWEEP_CASES:
        for _ in range(3):
            i += 1
            read = fixed + nrows * per_row + (weight if with_w else 0)
            rows.append((i, nrows * 512, "void arn::row_kernel<0>(arn::Args)", read, nrows * 8192))
    for _ in range(bench.COPY_REPS):
        i += 1
        rows.append((i, 1 << 20, "__amd_rocclr_copyBuffer", bench.COPY_BYTES, bench.COPY_BYTES))
    paths = {}
    for k, counter in ((3, "FETCH_SIZE"), (4, "WRITE_SIZE")):
        p = tmp_path / f"{counter}.csv"
        with open(p, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Grid_Size", "Kernel_Name",
                                              "Counter_Name", "Counter_Value"])
            w.writeheader()
            for r in rows:
                # the read counter reads half of the true bytes, in KiB
                v = r[k] / 1024 / (2 if k == 3 else 1)
                w.writerow({"Dispatch_Id": r[0], "Grid_Size": r[1], "Kernel_Name": r[2],
                            "Counter_Name": counter, "Counter_Value": v})
        paths[counter] = str(p)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    out = bench.summarize_launch_traffic(paths["FETCH_SIZE"], paths["WRITE_SIZE"])
    assert out["fit"]["read_bytes_per_row"] == pytest.approx(per_row)
    assert out["fit"]["read_fixed_bytes_per_launch"] == pytest.approx(fixed, abs=1)
    assert out["fit"]["read_weight_bytes_per_launch"] == [weight, weight]
    assert out["cases"][1]["write_bytes_per_launch"] == 65 * 8192
