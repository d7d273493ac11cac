"""CPU-only: builds libsvdq.so with the host translation units under
AddressSanitizer and UndefinedBehaviorSanitizer (g++), linked with the
ordinary device object, so the host half (preparation, packing, the
eigensolver, validation) can be run under the sanitizers:

    python w4a4_rank_corrected_smooth_amd/build.py          # device object
    python w4a4_rank_corrected_smooth_amd/build_sanitized.py
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1 \\
      LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)" \\
      python -m pytest tests -q -m "not gpu"
    python w4a4_rank_corrected_smooth_amd/build.py          # back to the normal library

The library it writes replaces the normal one in place; rebuild before any
GPU use.
"""
from __future__ import annotations

import os
import subprocess

import build as B

SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined"]


def main() -> None:
    dev = os.path.join(B.BUILD, "device.o")
    if not os.path.exists(dev):
        raise SystemExit("build the device object first: python w4a4_rank_corrected_smooth_amd/build.py")
    objs = []
    for src, extra in B.HOST_UNITS.items():
        obj = os.path.join(B.BUILD, src.replace(".cpp", ".san.o"))
        flags = [f for f in B.HOST_COMMON if f != "-O3"]
        subprocess.run(["g++", *SAN, *flags, *extra, "-c", os.path.join(B.CSRC, src), "-o", obj], check=True)
        objs.append(obj)
    subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", B.LIB, *objs, dev,
                    f"-L{B.ROCM}/lib", "-lamdhip64", "-lpthread", f"-Wl,-rpath,{B.ROCM}/lib"], check=True)
    print(B.LIB)


if __name__ == "__main__":
    main()
