"""bench.py's command-line contract that holds without a GPU: the path is
measured on exactly one GPU, so any other GPU count (or a multi-rank launch)
exits with status 2 and a message before any device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2, r.stderr
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_multi_rank_launch_is_refused():
    r = run_bench(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "4"})
    assert r.returncode == 2, r.stderr
    assert "exactly one GPU" in r.stderr
