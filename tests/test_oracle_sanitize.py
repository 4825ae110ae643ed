"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): tests/c/oracle_sanitize.c drives one small layer through forward
and backward in both weight formats; any out-of-bounds access or undefined
arithmetic aborts the run."""

import os
import shutil
import subprocess

import pytest

from .conftest import ROOT


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Wno-unknown-pragmas", "-o", str(exe),
                    os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "rawint4_oracle.c"), "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    print(run.stdout, run.stderr)
    assert run.returncode == 0, run.stderr
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
    assert run.stdout.count("rc=0 finite=1") == 2
