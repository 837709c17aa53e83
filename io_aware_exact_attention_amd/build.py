"""Build libfa355.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m io_aware_exact_attention_amd.build``.  The shared library is
written next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG_DIR, "csrc", "fa355.hip")
OUT = os.path.join(PKG_DIR, "libfa355.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-shared",
    "-fPIC",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libfa355")


# a C++ program that calls the library through the C ABI alone (host code; links libfa355.so)
EXAMPLE_SRC = os.path.join(PKG_DIR, "csrc", "c_example.cpp")
EXAMPLE_OUT = os.path.join(PKG_DIR, "fa355_c_example")


def _run(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stderr[-8000:])
    if verbose:
        noise = "packed-fp32-ops"
        for line in res.stderr.splitlines():
            if noise not in line:
                print(line)


def build(verbose: bool = False, extra_flags=None) -> str:
    _run([hipcc(), *HIPCC_FLAGS, *(extra_flags or []), SRC, "-o", OUT + ".tmp"], verbose)
    os.replace(OUT + ".tmp", OUT)
    _run([hipcc(), "-O2", "-std=c++17", EXAMPLE_SRC, "-o", EXAMPLE_OUT + ".tmp", "-L" + PKG_DIR,
          "-lfa355", "-Wl,-rpath,$ORIGIN"], verbose)
    os.replace(EXAMPLE_OUT + ".tmp", EXAMPLE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
