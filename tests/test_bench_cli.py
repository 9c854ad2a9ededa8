"""bench.py's command line (CPU): it measures one GPU and refuses any other count before touching a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, extra_env=None):
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    env.update(extra_env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = _run(["--gpus", str(n)])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus %d" % n in r.stderr
    assert r.stdout == ""                       # no JSON line for a run that did not happen


def test_launcher_world_size_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "--gpus 4 is not supported" in r.stderr
