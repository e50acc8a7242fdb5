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


def test_gemv_cpu_baseline_reads_the_layer_records():
    """The generation bench's oracle leg takes the same per-layer records as
    its timed steps (natural-order and act-order layers alike)."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import bench
    rng = np.random.default_rng(0)
    m, d, bits, group = 8, 256, 3, 128
    q = torch.from_numpy(rng.integers(-2 ** 31, 2 ** 31 - 1, (m, d * bits // 32), dtype=np.int64).astype(np.int32))
    sc = torch.rand(m, d // group) * 0.01 + 1e-3
    z = torch.randint(0, 8, (m, d // group), dtype=torch.uint8)
    x = torch.randn(d).half()
    y = torch.empty(m)
    perm = (torch.randperm(d).to(torch.int32), torch.empty(d, dtype=torch.float16))
    layers = [("a", q, sc, z, bits, group, x, y, 1000, None), ("b", q, sc, z, bits, group, x, y, 1000, perm)]
    out = bench.gemv_cpu_baseline(layers, rows=2)
    assert out["kind"] == "oracle" and out["value"] > 0 and out["unit"] == "tokens/s"
