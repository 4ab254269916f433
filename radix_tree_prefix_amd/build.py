"""Build librs.so (host radix tree + HIP kernels for gfx950) in-tree with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "librs.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["tree.cpp", "schedule.cpp", "draft.cpp", "plan.cpp", "kernels.hip", "hostpool.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # no packed-fp32 instructions in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


def build(verbose=False):
    """Compile every source (always) and link librs.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(len(cmds)) as ex:
        for r in ex.map(_run, cmds):
            if verbose and r.stderr:
                sys.stderr.write(r.stderr)
    tmp = OUT + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
