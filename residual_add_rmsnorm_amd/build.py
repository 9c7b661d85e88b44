"""Build libarn.so (HIP, gfx950 only) in-tree.

One object per operator kind and dtype is compiled from arn_kernels.hip,
arn_glu.hip and arn_gemm.hip (they build in parallel), plus the host
dispatcher arn_api.hip; hipcc links them into
residual_add_rmsnorm_amd/lib/libarn.so.  The streaming probe that measures
bandwidth ceilings (arn_probe.hip) becomes lib/libarn_probe.so, used only
by the benchmark.  The binding's per-call argument marshalling,
arn_pyext.cpp, is host C++ against torch's headers; g++ builds it into the
extension module lib/_native (no device code).

    python -m residual_add_rmsnorm_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import sysconfig
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libarn.so")
PROBE_LIB_PATH = os.path.join(LIB_DIR, "libarn_probe.so")
NATIVE_PATH = os.path.join(LIB_DIR, "_native" + sysconfig.get_config_var("EXT_SUFFIX"))
OBJ_DIR = os.path.join(ROOT, "_build", "arn")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32;
# ordinary scalar fp32 code is what the kernels are written as.
CFLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]

KINDS = range(6)
GLU_MODES = range(3)
DTYPES = range(2)


def sources() -> list[str]:
    return [os.path.join(CSRC, f) for f in ("arn_kernels.hip", "arn_glu.hip", "arn_gemm.hip",
                                            "arn_api.hip", "arn_internal.h", "arn_gemm.h", "arn_device.h",
                                            "arn_probe.hip", "arn_pyext.cpp")] + [
        os.path.join(INCLUDE, "arn.h"), os.path.join(INCLUDE, "arn_tuning.h"),
        os.path.join(INCLUDE, "arn_probe.h")]


def _compile(src: str, obj: str, defines: list[str]) -> None:
    cmd = [HIPCC, *CFLAGS, *defines, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so;
    # that note is expected.  Anything else is shown.
    noise = "packed-fp32-ops"
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({' '.join(cmd)}):\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)


def build_native() -> str:
    """The extension module holding the binding's argument marshalling."""
    import torch
    from torch.utils import cpp_extension

    torch_lib = os.path.join(os.path.dirname(torch.__file__), "lib")
    abi = int(torch._C._GLIBCXX_USE_CXX11_ABI)
    tmp = NATIVE_PATH + ".tmp"
    # hip_runtime_api.h (included by arn.h and torch's HIP stream header)
    # needs the platform named when a plain host compiler reads it.
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-fvisibility=hidden",
           "-Wall", "-Wno-unused-parameter", "-D__HIP_PLATFORM_AMD__",
           f"-D_GLIBCXX_USE_CXX11_ABI={abi}", "-DTORCH_EXTENSION_NAME=_native",
           f"-I{INCLUDE}", "-I/opt/rocm/include",
           *[f"-I{p}" for p in cpp_extension.include_paths()],
           f"-I{sysconfig.get_paths()['include']}",
           os.path.join(CSRC, "arn_pyext.cpp"), "-o", tmp,
           f"-L{torch_lib}", "-lc10", "-lc10_hip", "-ltorch_cpu", "-ltorch_python"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({' '.join(cmd)}):\n{res.stdout}{res.stderr}")
    if (res.stdout + res.stderr).strip():
        print(res.stdout + res.stderr, file=sys.stderr)
    os.replace(tmp, NATIVE_PATH)
    return NATIVE_PATH


def build(jobs: int | None = None, verbose: bool = True) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    units = []
    for k in KINDS:
        for d in DTYPES:
            units.append((os.path.join(CSRC, "arn_kernels.hip"),
                          os.path.join(OBJ_DIR, f"arn_kernels_k{k}_d{d}.o"),
                          [f"-DARN_KIND={k}", f"-DARN_DT={d}"]))
    for k in KINDS:
        for d in DTYPES:
            units.append((os.path.join(CSRC, "arn_kernels.hip"),
                          os.path.join(OBJ_DIR, f"arn_sum_k{k}_d{d}.o"),
                          [f"-DARN_KIND={k}", f"-DARN_DT={d}", "-DARN_SUM=1"]))
    for m in GLU_MODES:
        for d in DTYPES:
            units.append((os.path.join(CSRC, "arn_glu.hip"),
                          os.path.join(OBJ_DIR, f"arn_glu_m{m}_d{d}.o"),
                          [f"-DARN_GLU_MODE={m}", f"-DARN_DT={d}"]))
    for d in DTYPES:
        units.append((os.path.join(CSRC, "arn_gemm.hip"),
                      os.path.join(OBJ_DIR, f"arn_gemm_d{d}.o"), [f"-DARN_DT={d}"]))
    units.append((os.path.join(CSRC, "arn_api.hip"), os.path.join(OBJ_DIR, "arn_api.o"), []))
    probe = (os.path.join(CSRC, "arn_probe.hip"), os.path.join(OBJ_DIR, "arn_probe.o"), [])
    jobs = jobs or min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        native = ex.submit(build_native)
        list(ex.map(lambda u: _compile(*u), units + [probe]))
        native.result()
    tmp = PROBE_LIB_PATH + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, probe[1]],
                   check=True)
    os.replace(tmp, PROBE_LIB_PATH)
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[u[1] for u in units]]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


def is_stale() -> bool:
    built = (LIB_PATH, PROBE_LIB_PATH, NATIVE_PATH)
    if not all(os.path.exists(p) for p in built):
        return True
    t = min(os.path.getmtime(p) for p in built)
    return any(os.path.getmtime(s) > t for s in sources())


if __name__ == "__main__":
    build()
