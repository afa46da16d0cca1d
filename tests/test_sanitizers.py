"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two small drivers are built with gcc/g++ and the sanitizers, on the host only
(no device code is instrumented) and run here:

* the fp64 C oracle (``oracle/ssd_oracle.c``) on small ragged problems, every
  buffer allocated at its exact size, its functions cross-checked against each
  other (``tests/sanitize/oracle_driver.c``);
* the C ABI's argument validation, workspace sizing and chunk rule
  (``csrc/api.cpp`` compiled host-only and linked ahead of ``libssd.so``),
  driven through rejected calls with fake pointers that are never dereferenced
  (``tests/sanitize/abi_driver.cpp``).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
PKG = os.path.join(ROOT, "mamba_ssd_chunked_05_amd")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(exe, tmp_path, leaks):
    env = dict(os.environ, ASAN_OPTIONS=f"detect_leaks={int(leaks)}:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300, cwd=str(tmp_path))
    assert res.returncode == 0, f"{os.path.basename(exe)} failed:\n{res.stdout}\n{res.stderr[-4000:]}"
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    subprocess.run(["gcc", "-std=c11", *FLAGS, "-fopenmp", "-ffp-contract=off", "-o", exe,
                    os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-lm"],
                   check=True, capture_output=True, text=True)
    assert "all checks passed" in _run(exe, tmp_path, leaks=True)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers are not available")
def test_abi_validation_under_asan_ubsan(tmp_path):
    lib = os.path.join(PKG, "libssd.so")
    if not os.path.exists(lib):
        pytest.fail("libssd.so is not built (run mamba_ssd_chunked_05_amd/build.py)")
    exe = str(tmp_path / "abi_asan")
    subprocess.run(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-o", exe,
                    os.path.join(SAN, "abi_driver.cpp"), os.path.join(PKG, "csrc", "api.cpp"),
                    f"-L{PKG}", "-lssd", f"-Wl,-rpath,{PKG}", "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True, capture_output=True, text=True)
    # the instrumented copy of the ABI is the one the driver calls: it is defined in the executable
    syms = subprocess.run(["nm", "--defined-only", exe], capture_output=True, text=True, check=True).stdout
    assert " T ssd_forward_ex" in syms and "__asan_init" in subprocess.run(
        ["nm", exe], capture_output=True, text=True, check=True).stdout
    # the HIP runtime keeps allocations until exit: leak checking is off for this one
    assert "all checks passed" in _run(exe, tmp_path, leaks=False)
