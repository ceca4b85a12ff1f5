"""Host-side contract of bench.py that needs no GPU: the benchmark measures
one GPU and refuses any other GPU count before it touches a device."""
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), *args], cwd=REPO, env=env,
                          capture_output=True, text=True, timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), (["--gpus", "8", "--steps", "1"], {}),
                                      (["--gpus", "1"], {"WORLD_SIZE": "4"})],
                         ids=["gpus2", "gpus8", "world4"])
def test_more_than_one_gpu_is_refused(args, env):
    r = run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line for a refused run
