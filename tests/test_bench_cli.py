"""bench.py on the CPU: the per-phase algorithmic work adds up to the step's
stated total, and asking for more than one GPU exits with a message (there is no
multi-GPU path)."""

import os
import subprocess
import sys

from int4_quantized_moe_amd import workloads as W

from .conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_phase_work_adds_up_to_the_step():
    for cfg in W.CONFIGS:
        slots = cfg.qlen * cfg.top_k
        work = bench.phase_work(cfg, slots)
        total = sum(f for f, _ in work.values())
        H, I, r = cfg.hidden, cfg.intermediate, cfg.rank
        assert total == slots * (12 * H * I + 18 * r * (H + I)), cfg.name
        proj = H * I // 2 + H * I // 16
        assert sum(b for _, b in work.values()) == 6 * proj  # two passes over three projections


def test_more_than_one_gpu_is_refused():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert run.returncode == 2 and "one GPU" in run.stderr
