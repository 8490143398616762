"""bench.py refuses multi-GPU runs (CPU only): with --gpus above 1, or under a
launcher that sets WORLD_SIZE above 1, it exits with status 2 and a message
before touching a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU only" in r.stderr
