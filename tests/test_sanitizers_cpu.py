"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: the oracle (every entry point, seeded inputs and edge cases, buffers
of exact size) and the C ABI's host side (argument refusals, empty calls,
size queries, tuning knobs, the plan buffer) must run without a report.
The drivers live in tests/sanitize/; device code is never sanitized (GPU
sanitizers are not used here)."""
import os
import shutil
import subprocess

import pytest

from tests.sanitize import build as san

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    report = res.stderr
    assert "AddressSanitizer" not in report and "runtime error" not in report, report
    assert res.returncode == 0, report
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_sanitizer_is_live(tmp_path):
    """A planted heap overflow in a throwaway program must be reported, so a
    clean run below means something."""
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\nint main(void) { int *p = malloc(4 * sizeof(int));"
                   " p[4] = 1; free(p); return 0; }\n")
    exe = tmp_path / "overflow"
    subprocess.run(["gcc", "-g", *san.SAN, str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60, env=ENV)
    assert res.returncode != 0 and "heap-buffer-overflow" in res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers():
    assert "all calls clean" in _run(san.oracle_driver())


@pytest.mark.skipif(not os.path.exists(os.path.join(san.ROCM, "llvm", "bin", "clang++")),
                    reason="needs ROCm's clang++")
def test_abi_host_code_under_sanitizers():
    assert "all calls clean" in _run(san.abi_driver())
