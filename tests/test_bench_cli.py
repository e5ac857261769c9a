"""bench.py's command line on the host: a request for more than one GPU is
refused with a message and exit status 2, before any device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_launcher_world_size_is_refused():
    env = dict(os.environ, WORLD_SIZE="8")
    r = run_bench(env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
