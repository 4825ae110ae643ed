"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C ABI source (argument checks, workspace planning, launch bookkeeping,
metadata) is compiled for the host alone with both sanitizers and linked with
the library's kernel objects from the ordinary build; tests/c/abi_sanitize.c
then sweeps the workspace planner up to the ABI's limits and drives every entry
point through its argument errors, all answered on the host (no GPU needed).
Any out-of-bounds access, leak or undefined arithmetic aborts the run.
"""

import glob
import os
import shutil
import subprocess

import pytest

from int4_quantized_moe_amd import build as hip_build

from .conftest import ROOT

HIPCC = hip_build.HIPCC
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host",
       "-fno-sanitize-recover=all"]


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("gcc") is None, reason="needs hipcc and gcc")
def test_library_host_code_clean_under_sanitizers(tmp_path):
    kernels = [os.path.join(hip_build.OBJDIR, os.path.basename(s) + ".o")
               for s in sorted(glob.glob(os.path.join(hip_build.CSRC, "*.hip"))) if not s.endswith("kt_api.hip")]
    if not all(os.path.exists(o) for o in kernels):
        hip_build.build()
    api = tmp_path / "kt_api_san.o"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "--offload-host-only", "-O1", "-g", "-std=c++17",
                    "-fno-omit-frame-pointer", *SAN, "-I" + os.path.join(ROOT, "include"), "-c",
                    os.path.join(hip_build.CSRC, "kt_api.hip"), "-o", str(api)], check=True, capture_output=True)
    driver = tmp_path / "abi_sanitize.o"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-c",
                    os.path.join(ROOT, "tests", "c", "abi_sanitize.c"), "-o", str(driver)], check=True)
    exe = tmp_path / "abi_sanitize"
    subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN[:4], str(api), *kernels, str(driver), "-o", str(exe)],
                   check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout[-3000:], run.stderr[-3000:])
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
    assert "FAIL" not in run.stdout and ", 0 failed" in run.stdout
