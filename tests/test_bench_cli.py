"""CPU: the benchmark's command-line contract that needs no GPU.

bench.py measures one GPU; asked for more it must stop with a message and a
non-zero status before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    p = _run(env=env)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
