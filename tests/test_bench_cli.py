"""bench.py's host-side argument rules, checked before it touches a GPU:
one GPU only (a multi-GPU request exits with status 2 and says so), no
HIP-graph capture of the three-launch prolog, and --graph-steps dividing
the step counts."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120, env=e)


@pytest.mark.parametrize("args,env,needle", [
    (("--gpus", "2"), None, "one GPU only"),
    (("--gpus", "8"), None, "one GPU only"),
    ((), {"WORLD_SIZE": "2"}, "one GPU only"),
    (("--graph", "--separate-prolog"), None, "drop --separate-prolog"),
    (("--graph", "--graph-steps", "3", "--steps", "10"), None, "--graph-steps must divide"),
    (("--graph", "--graph-steps", "0"), None, "--graph-steps must divide"),
])
def test_rejected_before_any_gpu_work(args, env, needle):
    r = _run(*args, env=env)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert needle in r.stderr
    assert r.stdout.strip() == ""   # no JSON line
