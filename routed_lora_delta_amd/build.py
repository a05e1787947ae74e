"""Build librld.so (HIP C++ for gfx950) in-tree with hipcc.

    python routed_lora_delta_amd/build.py [-v]

(run by path: importing the package itself needs the library this builds).

Every call recompiles every source.  Objects go to routed_lora_delta_amd/_build/,
the library to routed_lora_delta_amd/librld.so.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librld.so")
ARCH = "gfx950"

# Packed fp32 ops stay off: hipcc would otherwise form v_pk_* fp32 forms by itself.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall",
          "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librld.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, "-x", "hip", *DEVICE_FLAGS, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + _filter(res.stderr))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def _filter(err: str) -> str:
    # the host pass does not know the device-only feature; that note is harmless
    return "".join(l + "\n" for l in err.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + _filter(res.stderr))
    if res.returncode != 0:
        raise RuntimeError("linking librld.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
