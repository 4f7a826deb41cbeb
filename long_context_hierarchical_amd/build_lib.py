"""Compile the RecSA HIP library (librecsa.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "librecsa.so")
SOURCES = ["build_tree.hip", "step.hip", "attend.hip", "backward.hip", "distill.hip", "dense.hip", "two_stage.hip",
           "noalloc.hip", "rope_cache.hip", "api.cpp"]
# HBM read/copy probe (a separate program, not part of the library): the achievable bandwidth
PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE = os.path.join(PKG, "probe", "hbm_probe")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # every multiply-add the kernels want fused is written as fmaf(); the rest must round twice
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int | None = None) -> str:
    from concurrent.futures import ThreadPoolExecutor
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        cmds.append([cc, *COMMON, "-c", path, "-o", obj])
        objs.append(obj)
    # the translation units are independent: compile them side by side
    n = jobs or max(1, min(len(cmds), len(os.sched_getaffinity(0)), 16))

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    with ThreadPoolExecutor(n) as ex:
        list(ex.map(run, cmds))
    tmp = OUT + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    cmd = [cc, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", PROBE_SRC, "-o", PROBE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(PROBE + ".tmp", PROBE)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
