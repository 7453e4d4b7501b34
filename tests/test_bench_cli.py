"""bench.py's command line on the CPU: it measures one GPU, so any request
for more (the flag or a launcher's WORLD_SIZE) ends with exit status 2 and a
message, before any device or library is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, **env):
    e = dict(os.environ, **env)
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=e, capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run(args, **env)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_workload_flag():
    r = _run(["--help"])
    assert r.returncode == 0
    assert "--workload" in r.stdout and "--gpus" in r.stdout and "--ramp" in r.stdout
