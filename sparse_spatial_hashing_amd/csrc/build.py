"""Build the gfx950 library in-tree: ``python sparse_spatial_hashing_amd/csrc/build.py``.

A standalone script (the package itself refuses to import without the library).

Flags: -O3, no fast-math (binning must be IEEE fp32), no FMA contraction,
packed-FP32 instructions disabled, position-independent shared object.
"""
from __future__ import annotations

import os
import subprocess
import sys

CSRC = os.path.dirname(os.path.abspath(__file__))
HERE = os.path.dirname(CSRC)
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(CSRC, "voxelize.hip"), os.path.join(CSRC, "spherical.hip")]
SOURCE = SOURCES[0]
HEADER = os.path.join(ROOT, "include", "voxelize.h")
LIBRARY = os.path.join(HERE, "libvoxelize.so")
ARCH = os.environ.get("VOX_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC", "-shared", "-Wall",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(output: str = LIBRARY, quiet: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.dirname(HEADER), "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{msgs}")
    if msgs.strip() and not quiet:
        print(msgs, file=sys.stderr)
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    print(build())
