"""The benchmark's argument checks (CPU only: every case below exits before
any GPU work): one GPU only, and the three-tier option only where that
variant is built (the MX format's forward with per-query-block budgets)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr


@pytest.mark.parametrize("extra", [["--fmt", "nvfp4"], ["--pass", "bwd"], ["--budget", "head"],
                                   ["--workload", "decode"]])
def test_three_tier_option_outside_its_variant_is_refused(extra):
    r = _run("--tier8-bp", "1000", *extra)
    assert r.returncode == 2 and "--tier8-bp" in r.stderr
