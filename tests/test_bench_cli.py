"""bench.py's command line on a host: the multi-GPU request is refused, and without a GPU the
benchmark stops with an error instead of measuring anything else."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert r.stdout.strip() == "" or not r.stdout.lstrip().startswith("{")  # no JSON line


def test_no_gpu_is_an_error():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert "no GPU" in r.stdout + r.stderr
