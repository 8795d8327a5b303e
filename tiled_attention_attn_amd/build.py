"""Builds the HIP library ``libtiled_attn.so`` for gfx950, in the package directory.

Every ``csrc/*.hip`` file is compiled to an object with hipcc (in parallel),
then linked into one shared library that exports the C ABI of
``include/tiled_attn.h``.  Packed-FP32 instruction selection is turned off for
the device code (``-packed-fp32-ops``).
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
OUT = os.path.join(PKG, "libtiled_attn.so")
OBJ_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("TATTN_OFFLOAD_ARCH", "gfx950")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "argument unused during compilation")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libtiled_attn.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_run, [hipcc, *COMMON, "-c", s, "-o", o]) for s, o in zip(srcs, objs)]
        for f in futs:
            msg = f.result()
            if verbose and msg:
                print(msg, file=sys.stderr)
    tmp = OUT + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
