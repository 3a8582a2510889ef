"""Build libh3a.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m store_kvi8r_quantize_amd.build

Every source is compiled to an object in parallel, then linked into
store_kvi8r_quantize_amd/lib/libh3a.so.  Always rebuilds.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libh3a.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no reassociation or contraction beyond what the sources write explicitly
    "-ffp-contract=off",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(OBJ_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OBJ_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = [[cc, *FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(min(8, len(jobs))) as ex:
        logs = list(ex.map(_run, jobs))
    tmp = LIB_PATH + ".tmp"
    logs.append(_run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB_PATH)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
