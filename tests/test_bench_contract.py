"""bench.py's command-line contract that needs no GPU: it measures one GPU
and refuses more, before touching the device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=e)


def test_more_than_one_gpu_is_refused():
    r = run(["--gpus", "2"])
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""


def test_a_distributed_launch_is_refused():
    r = run(["--gpus", "1"], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "single GPU" in r.stderr and r.stdout == ""
