"""Compile the HIP sources into ``libspec_verify.so`` (in-tree, gfx950)."""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspec_verify.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # Keep the compiler from emitting packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def build(force: bool = True, extra_flags: list[str] | None = None) -> str:
    """Build ``libspec_verify.so`` next to this file and return its path."""
    if not force and os.path.exists(LIB):
        return LIB
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include")] + list(extra_flags or [])
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        procs.append(subprocess.Popen([hipcc(), *flags, "-c", src, "-o", obj]))
    for p, src in zip(procs, srcs):
        if p.wait() != 0:
            raise RuntimeError(f"hipcc failed on {src}")
    tmp = LIB + ".tmp"
    subprocess.run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
