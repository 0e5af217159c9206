"""bench.py command line: it measures one GPU and refuses more, before it
touches torch or a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=60, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""


def test_a_distributed_launch_is_refused_too():
    env = dict(os.environ, WORLD_SIZE="8")
    r = _run([], env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
