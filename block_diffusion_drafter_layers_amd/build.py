"""Build the HIP library ``libdflash.so`` in-tree for gfx950.

    python -m block_diffusion_drafter_layers_amd.build

Every ``csrc/*.hip`` file is compiled by hipcc (in parallel) to an object
under ``_build/`` and linked into ``block_diffusion_drafter_layers_amd/libdflash.so``.
Cross-compiles without a GPU.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdflash.so")
ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that noise
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln)
    return msg


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(16, os.cpu_count() or 1)

    def compile_one(pair):
        src, obj = pair
        out = _run([HIPCC, *CFLAGS, "-c", src, "-o", obj])
        if verbose and out.strip():
            print(out, file=sys.stderr)

    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
