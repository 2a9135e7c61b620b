"""Builds libstdk.so (the HIP library) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "api.hip")
LIB = os.path.join(HERE, "libstdk.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libstdk.so)")


def build(verbose: bool = True) -> str:
    """Compile csrc/api.hip (which includes every kernel) into libstdk.so.
    Always recompiles; the new library replaces the old one atomically."""
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp, SRC]
    if verbose:
        print("[stdk build]", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
