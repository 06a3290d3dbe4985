"""Builds libmoe_overlap.so in-tree: the gfx950 kernels and the C ABI.

Every HIP source is compiled for gfx950 only, with packed fp32 arithmetic
disabled, then linked with the host-only partition model into one shared
library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libmoe_overlap.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIP_SOURCES = ["route.hip", "permute.hip", "gemm.hip", "consumer.hip", "combine.hip", "partition.hip",
               "abi.hip"]
CXX_SOURCES = []

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INC, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-I", INC, "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the gfx feature flag: harmless, filter it
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False, jobs: int = 8, defines=(), out: str = OUT, build_dir: str = BUILD) -> str:
    """Compiles and links the library; `defines` are extra -D flags (e.g. for
    tuning variants built to another `out` path)."""
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        cmds.append([HIPCC, *HIP_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        cmds.append(["g++", *CXX_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, log) in zip(cmds, results):
        if log.strip() and (verbose or rc != 0):
            print(log, file=sys.stderr)
        if rc != 0:
            failed = True
            print(f"FAILED: {' '.join(cmd)}", file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed")
    tmp = out + ".tmp"
    rc, log = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    if rc != 0:
        print(log, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("-D", action="append", default=[], help="extra preprocessor define")
    ap.add_argument("--out", default=OUT)
    ap.add_argument("--build-dir", default=BUILD)
    a = ap.parse_args()
    print(build(verbose=a.v, defines=a.D, out=a.out, build_dir=a.build_dir))
