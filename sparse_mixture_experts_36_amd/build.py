"""Builds libmoe.so (the gfx950 HIP library behind include/moe.h) in-tree.

    python -m sparse_mixture_experts_36_amd.build [-v]

Every kernel source is compiled for gfx950 only. Packed fp32 instructions are
switched off for device code (they are generated from ordinary float code at
-O3 and are avoided here on purpose); the host pass warns that it does not
know that feature, which is harmless.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-I", os.path.join(ROOT, "include"), "-I", CSRC] + DEVICE_FLAGS
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = common + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp"
    link = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if p.returncode != 0:
        sys.stderr.write(text)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}")
    if lines and os.environ.get("MOE_BUILD_VERBOSE"):
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
