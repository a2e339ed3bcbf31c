"""Builds libmoe.so (the HIP kernels and the C ABI of include/moe.h) for gfx950, in-tree."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmoe.so")
OBJ = os.path.join(ROOT, "_build")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: plain fp32 code is compiled to scalar-pair ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # register-staged tiles must stay in registers, never be moved to LDS
    "-mllvm", "-disable-promote-alloca-to-lds",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, out: str = OUT, defines=(), obj_dir: str = OBJ) -> str:
    """Compile every csrc/*.hip and link `out`. `defines` (NAME=VALUE strings) select
    compile-time tile shapes; the defaults are the tuned ones."""
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    objs = []
    for s in srcs:
        o = os.path.join(obj_dir, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + ["-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = False
    for s, p in procs:
        log, _ = p.communicate()
        text = "\n".join(l for l in log.decode().splitlines()
                         if "packed-fp32-ops" not in l)
        if text.strip():
            print(text, file=sys.stderr)
        if p.returncode != 0:
            failed = True
            print(f"hipcc failed on {s}", file=sys.stderr)
    if failed:
        raise RuntimeError("HIP build failed")
    tmp = out + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp],
                   check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
