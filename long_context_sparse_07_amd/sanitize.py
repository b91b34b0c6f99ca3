"""Host-sanitizer build of the C ABI's validation and dispatch code (csrc/api.cpp).

api.cpp is compiled by g++ with AddressSanitizer and UndefinedBehaviorSanitizer (host
code only: no device code is built here) and linked with the ordinary kernel objects
of the in-tree build into _build/sanitize/liblsa_sanitized.so. The CPU test
tests/test_abi_sanitized.py runs the ABI host tests against it (LSA_LIB_PATH), with the
ASan runtime preloaded into the Python process.

Usage: python -m long_context_sparse_07_amd.sanitize
"""
from __future__ import annotations

import os
import subprocess
import sys

from long_context_sparse_07_amd import build as B

OUT = os.path.join(B.BUILD, "sanitize")
LIB = os.path.join(OUT, "liblsa_sanitized.so")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """The g++ ASan runtime (to preload into an uninstrumented Python)."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def build_sanitized() -> str:
    os.makedirs(OUT, exist_ok=True)
    objs = [os.path.join(B.BUILD, os.path.basename(s) + ".o") for s in B.sources() if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    api = os.path.join(B.CSRC, "api.cpp")
    api_o = os.path.join(OUT, "api.o")
    inc = ["-I", os.path.join(B.ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]
    cc = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN, *inc, "-c", api, "-o", api_o]
    r = subprocess.run(cc, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile of api.cpp failed:\n{r.stderr}")
    ld = ["g++", "-shared", *SAN, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib",
          "-o", LIB]
    r = subprocess.run(ld, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return LIB


if __name__ == "__main__":
    print(build_sanitized())
    sys.exit(0)
