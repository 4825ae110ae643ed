"""The C ABI from plain C: tests/c/abi_consumer.c is compiled with gcc against
include/kt_rawint4.h, linked to the built library and run (host checks only, no
GPU calls)."""

import os
import shutil
import subprocess

import pytest

from int4_quantized_moe_amd import _lib

from .conftest import ROOT


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_consumer(tmp_path):
    lib_dir = os.path.dirname(_lib.LIBRARY_PATH)
    exe = tmp_path / "abi_consumer"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_consumer.c"), "-o", str(exe), "-L", lib_dir,
                    "-l:libkt_rawint4.so", f"-Wl,-rpath,{lib_dir}", "-lm"], check=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "FAIL" not in run.stdout and run.stdout.count("ok") >= 12
