"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a device (the library has no multi-GPU path)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, **(env or {})))


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
