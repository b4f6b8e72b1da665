"""Build libmoe.so (the C-ABI library of HIP kernels for gfx950) in-tree.

Usage: python -m routing_dispatch_expert_logits_amd.build [-v]

Every source under csrc/ is compiled by hipcc for gfx950 only, in parallel,
then linked into routing_dispatch_expert_logits_amd/libmoe.so.  Packed fp32
ALU ops are disabled for the device code (-packed-fp32-ops): plain fp32 math
only.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -amdgpu-atomic-optimizer-strategy=None: the optimizer turns a one-lane atomic with a
# uniform address (the persistent GEMM's tile claim) into a combine that waits for the
# result at once, which drains the claiming loader wave's LDS DMA stages.
DEVICE_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
                "-Wall", "-Wno-unused-function", "-fvisibility=hidden",
                "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and noise not in ln]
    if msgs and verbose:
        print("\n".join(msgs))
    return r


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in sources():
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *DEVICE_FLAGS, "-c", src, "-o", obj])
    with ThreadPoolExecutor(jobs) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
