"""The C ABI's host code (validation, sizing, workspace carving, launch planning of api.cpp) built
with AddressSanitizer and UndefinedBehaviorSanitizer by g++, with the kernel launchers replaced by
host stand-ins (tests/sanitize/launch_stubs.cpp), and driven through every entry point by
tests/sanitize/abi_driver.cpp (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "nvfp4_block_scaled_mxfp8_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = "/opt/rocm"
FLAGS = ["-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include"),
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
                    reason="needs g++ and the HIP runtime library")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libgmlp_host_san.so")
    hip = ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    _run(["g++", "-fPIC", "-shared"] + FLAGS + [os.path.join(CSRC, "api.cpp"), os.path.join(SAN, "launch_stubs.cpp"),
                                               "-o", lib] + hip)
    drv = str(tmp_path / "abi_driver")
    _run(["g++"] + FLAGS + [os.path.join(SAN, "abi_driver.cpp"), "-L" + str(tmp_path), "-lgmlp_host_san",
                            "-Wl,-rpath," + str(tmp_path), "-o", drv] + hip)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([drv], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in out and "runtime error" not in out and "LeakSanitizer" not in out, out
    assert "all statuses as expected" in out
