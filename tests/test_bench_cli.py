"""bench.py measures one GPU: asked for more (by flag or by a multi-rank
launcher's WORLD_SIZE) it exits with status 2 and says why, before touching a
device.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, BENCH] + args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=300)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = _run(["--gpus", str(n), "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_multi_rank_launch_is_refused():
    r = _run(["--steps", "1", "--warmup", "0"], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
