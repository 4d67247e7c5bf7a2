"""bench.py's command-line contract on a host without a GPU: more than one
GPU is refused with a message (this path has no sharded mode), and with no
HIP device the run fails with a non-zero status instead of falling back to
anything else."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = _run(["--gpus", str(n)])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_no_device_fails_loudly():
    if os.path.exists("/dev/kfd"):
        pytest.skip("a HIP device may be present")
    r = _run(["--steps", "1", "--warmup", "0"])
    assert r.returncode != 0
    assert "HIP device" in r.stderr
    assert r.stdout.strip() == ""
