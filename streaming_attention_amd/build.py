"""Build step: compile the HIP sources for gfx950 into ``libattn.so`` in-tree.

Usage: ``python -m streaming_attention_amd.build`` (or ``build()`` from Python).
Every call recompiles.  Objects go to ``_build/`` (not committed); the shared
library lands next to this file, where the binding loads it.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the GPU-only target feature; that warning is harmless.
    out = "\n".join(ln for ln in r.stdout.splitlines()
                    if "packed-fp32-ops" not in ln and "unknown target feature" not in ln
                    and ln.strip() and not ln.strip().startswith("1 warning"))
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_run, [hipcc, *COMMON_FLAGS, "-c", s, "-o", ob]) for s, ob in zip(srcs, objs)]
        for f in futs:
            out = f.result()
            if verbose and out:
                print(out)
    tmp = LIB + f".tmp{os.getpid()}"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
