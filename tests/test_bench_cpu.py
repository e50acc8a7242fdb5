"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message (the benchmark measures one GPU), and --static-groups needs
--act-order. Neither path touches a GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_static_groups_need_act_order():
    p = _run("--static-groups")
    assert p.returncode == 2
    assert "--act-order" in p.stderr
    assert p.stdout.strip() == ""
