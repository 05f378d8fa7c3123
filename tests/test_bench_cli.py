"""CPU checks of bench.py's command line: it runs on one GPU only and says so
(exit status 2) before touching a GPU when asked for more."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_exits_with_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_distributed_launch_exits_with_message():
    r = _run(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_help_lists_modes():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--workload", "--sweep", "--backward-sweep", "--mla-sweep", "--backward", "--mla",
                 "--copy-calibration", "--no-cpu-baseline"):
        assert flag in r.stdout
