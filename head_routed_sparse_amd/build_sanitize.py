"""Host-sanitizer build of the library for the CPU tests: the host code (hc_api.cpp:
argument validation, layout, ring bookkeeping, planning, host reductions) compiled by
g++ with AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts), linked
with the kernel objects of the regular gfx950 build (their device code is not
instrumented). Writes _build/sanitize/libheadcast_san.so.

Run the host tests against it with the sanitizer runtime preloaded (python itself is
not instrumented), as tests/test_host_sanitizers.py does:
    HEADCAST_LIBRARY=<that .so> LD_PRELOAD=<libasan.so> ASAN_OPTIONS=detect_leaks=0 \\
        python -m pytest tests/test_host_abi.py
"""
from __future__ import annotations

import os
import subprocess
import sys

from head_routed_sparse_amd import build as hb

OUT = os.path.join(hb.BUILD, "sanitize")
LIB = os.path.join(OUT, "libheadcast_san.so")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """Path of the compiler's ASan runtime (to preload)."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build() -> str:
    objs = [os.path.join(hb.BUILD, os.path.splitext(s)[0] + ".o") for s in hb.SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        hb.build()
    os.makedirs(OUT, exist_ok=True)
    api = os.path.join(OUT, "hc_api.o")
    host = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN]
    subprocess.run([*host, "-c", os.path.join(hb.CSRC, "hc_api.cpp"), "-o", api], check=True)
    subprocess.run(["g++", "-shared", *SAN, "-o", LIB, api, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib"], check=True)
    return LIB


if __name__ == "__main__":
    print(build(), file=sys.stderr)
