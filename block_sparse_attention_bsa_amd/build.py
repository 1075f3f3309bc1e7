"""Build libbsa.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_bsa_amd.build

Compiles every source each time it runs (objects go to _build/ at the repo
root, the library next to this file).
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsa.so")

ARCH = "gfx950"
DEVICE_SOURCES = ["bsa_fwd.hip", "bsa_fwd_pp.hip", "bsa_fwd_staged.hip", "bsa_meta.hip",
                  "bsa_bwd.hip", "bsa_bwd_proxy.hip"]
HOST_SOURCES = ["bsa_api.cpp"]
# Packed fp32 VALU forms are kept out of the device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsa.so)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; drop that notice
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = True, jobs: int = 4) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    steps = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append((obj, [hipcc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append((obj, [hipcc, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        outs = list(ex.map(lambda s: _run(s[1]), steps))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [s[0] for s in steps])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, jobs=int(sys.argv[1]) if len(sys.argv) > 1 else 4)
