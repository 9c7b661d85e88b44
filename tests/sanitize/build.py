"""Build the host-code sanitizer drivers (CPU only, no GPU needed).

* oracle_driver: oracle/oracle.c and oracle_driver.c, gcc with
  AddressSanitizer and UndefinedBehaviorSanitizer.
* abi_driver: the host code of residual_add_rmsnorm_amd/csrc/arn_api.hip
  compiled by hipcc with the sanitizers on the host pass only (each
  -fsanitize= behind -Xarch_host; device code is built as usual), linked
  by ROCm's clang++ with abi_driver.c and the library's kernel objects
  from the regular build.

Outputs go to _build/sanitize/.  Each build raises on a compiler error and
returns the executable's path.
"""
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CSRC = os.path.join(ROOT, "residual_add_rmsnorm_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)} failed:\n{res.stdout}{res.stderr}")


def oracle_driver() -> str:
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", *SAN,
          "-I", os.path.join(ROOT, "oracle"), os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-o", exe])
    return exe


def abi_driver() -> str:
    from residual_add_rmsnorm_amd import build as lib_build

    if lib_build.is_stale():
        lib_build.build(verbose=False)
    os.makedirs(OUT, exist_ok=True)
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    api_obj = os.path.join(OUT, "arn_api_san.o")
    host_san = []
    for flag in SAN:
        host_san += ["-Xarch_host", flag]
    _run([hipcc, "-O1", "-g", f"--offload-arch={lib_build.ARCH}", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *host_san,
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", "-c",
          os.path.join(CSRC, "arn_api.hip"), "-o", api_obj])
    drv_obj = os.path.join(OUT, "abi_driver.o")
    _run([clangxx, "-x", "c", "-O1", "-g", "-std=c11", *SAN, "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), "-c",
          os.path.join(HERE, "abi_driver.c"), "-o", drv_obj])
    kernels = [o for o in glob.glob(os.path.join(lib_build.OBJ_DIR, "*.o"))
               if os.path.basename(o) not in ("arn_api.o", "arn_probe.o")]
    exe = os.path.join(OUT, "abi_driver")
    _run([clangxx, *SAN, drv_obj, api_obj, *kernels, "-L", os.path.join(ROCM, "lib"),
          "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe])
    return exe
