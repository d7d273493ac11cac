"""Builds libsvdq.so in-tree: host translation units with g++, the device
translation unit with hipcc for gfx950, linked into one shared library next
to this file.  Usable without torch or a built library:  python w4a4_rank_corrected_smooth_amd/build.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsvdq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HOST_COMMON = ["-O3", "-std=c++17", "-fPIC", "-mavx2", "-mfma", "-Wall", "-Wno-unknown-pragmas",
               f"-I{INCLUDE}", f"-I{CSRC}"]
# Files whose float32 results must be reproducible bit for bit never fuse
# multiply-add; the dense float64 algebra may.
HOST_UNITS = {
    "abi_host.cpp": ["-ffp-contract=off"],
    "host_prepare.cpp": ["-ffp-contract=off"],
    "host_threads.cpp": [],
    "host_linalg.cpp": ["-ffp-contract=fast"],
}
DEVICE_UNITS = ["device.hip"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    lines = [l for l in out.splitlines() if "is not a recognized feature for this target" not in l]
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


def build(verbose: bool = False) -> str:
    """Compile every source and link libsvdq.so.  Always recompiles."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src, extra in HOST_UNITS.items():
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        _run(["g++", *HOST_COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    for src in DEVICE_UNITS:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([hipcc, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread",
          f"-Wl,-rpath,{ROCM}/lib"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
