"""Build of the HIP library libmoe_mi355x.so (gfx950), in-tree.

Compiles every .hip source under csrc/ with hipcc for gfx950 and links one
shared library next to this file.  Packed-fp32 instruction selection is
turned off for device code (the layer's fp32 arithmetic uses ordinary
v_fma/v_mul/v_add).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-mllvm", "-disable-promote-alloca-to-lds",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(os.path.dirname(HERE), "include")]


# Extra hipcc flags per source file.
PER_FILE = {
    "gemm.hip": os.environ.get("MOE_GEMM_FLAGS", "-mllvm -amdgpu-sched-strategy=iterative-minreg").split(),
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [
        os.path.join(os.path.dirname(HERE), "include", "moe.h")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + PER_FILE.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    if out.strip():
        print(out)
    return obj


def build(force: bool = True) -> str:
    """Compile and link; returns the library path."""
    srcs = sources()
    if not force and os.path.exists(LIB):
        newest = max(os.path.getmtime(p) for p in srcs + headers())
        if os.path.getmtime(LIB) >= newest:
            return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
