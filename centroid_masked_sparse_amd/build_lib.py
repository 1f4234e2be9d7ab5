"""Build ``libce.so`` (HIP kernels + C-ABI host library) for gfx950 in-tree.

Usage: ``python -m centroid_masked_sparse_amd.build_lib`` or ``build()``.
The library is written next to this file; object files go to ``_build/`` at
the repository root.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libce.so")
SOURCES = ("ce_kernels.hip", "ce_host.cpp")
ARCH = "gfx950"

# Packed fp32 arithmetic is switched off for all device code; the host pass
# warns that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")
    return r


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libce.so``; returns its path."""
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              f"-I{os.path.join(ROOT, 'include')}", *DEVICE_FLAGS]
    objs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        _run([_hipcc(), *common, "-c", os.path.join(HERE, "csrc", src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    _run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
