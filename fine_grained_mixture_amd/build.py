"""Builds libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m fine_grained_mixture_amd.build   (or __graft_entry__.build())
Object files go to fine_grained_mixture_amd/_build/; the library is written
to fine_grained_mixture_amd/libmoe.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")

SOURCES = ["moe_api.hip", "route.hip", "gemm_fwd.hip", "gemm_bwd.hip", "aggregate.hip",
           "router.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU ops stay off; hipcc's host pass warns that it does not
    # know the feature, which is harmless.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int | None = None, lib: str = LIB,
          objdir: str = OBJDIR) -> str:
    """Compiles every source and links `lib`."""
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.rsplit(".", 1)[0] + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for cmd, msg in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(" ".join(cmd[-3:]), file=sys.stderr)
            if msg.strip() and verbose:
                print(msg, file=sys.stderr)
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
