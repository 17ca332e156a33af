"""bench.py on the host: it runs on exactly one GPU and refuses anything else
before touching a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_a_distributed_launch_is_refused_too():
    r = run_bench([], {"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "WORLD_SIZE=8" in r.stderr
