"""bench.py's command-line contract on the host: more than one GPU is refused
with a message before torch or the GPU is touched, and unknown workloads are
argument errors."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = run_bench("--gpus", str(n), "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_distributed_launch_is_refused():
    r = run_bench("--gpus", "1", env_extra={"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr
    assert r.stdout == ""


def test_unknown_workload_is_an_argument_error():
    r = run_bench("--workload", "no-such-workload")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr
