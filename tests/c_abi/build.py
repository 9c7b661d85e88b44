"""Compile arn_client.c (host C, gcc) against include/arn.h and libarn.so.

The client lives next to the tests that run it; build() of the repository
compiles it with everything else, and the test compiles it only if it is
missing or older than its source or the header.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "arn_client.c")
EXE = os.path.join(HERE, "arn_client")
LIB_DIR = os.path.join(ROOT, "residual_add_rmsnorm_amd", "lib")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", LIB_DIR, "-larn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../residual_add_rmsnorm_amd/lib",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", EXE + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


def ensure() -> str:
    header = os.path.join(ROOT, "include", "arn.h")
    if not os.path.exists(EXE) or os.path.getmtime(EXE) < max(os.path.getmtime(SRC),
                                                               os.path.getmtime(header)):
        build()
    return EXE
