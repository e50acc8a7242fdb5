"""Build libgptq_mi355x.so (gfx950) in-tree with hipcc.

    python -m post_weight_quantization_18_amd.build

Each .hip source is compiled to an object under _build/ (in parallel) and the
objects are linked into post_weight_quantization_18_amd/libgptq_mi355x.so.
Packed fp32 instructions are disabled on purpose (-packed-fp32-ops).
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgptq_mi355x.so")
SOURCES = ["gptq_api.hip", "syrk.hip", "chain.hip", "quant.hip", "trail.hip", "order.hip", "gemv.hip", "trace.hip",
           "colloop_row.hip", "colloop_g16.hip", "colloop_g32.hip", "colloop_g64.hip", "colloop_g128.hip", "colloop_wide.hip",
           "colloop_static.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-Werror=inline-asm", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (p.stdout + p.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
