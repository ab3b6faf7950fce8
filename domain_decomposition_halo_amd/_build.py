"""Compile the HIP library libddh.so for gfx950 (in-tree)."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libddh.so")
SOURCES = ["ddh_api.hip", "ddh_build.hip", "ddh_exchange.hip"]

# -ffp-contract=off: every fp32 add and multiply is one rounded IEEE operation,
# as the bit-exact results require. Packed fp32 instructions are disabled.
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]
# named host ranges of the entry points for rocprofv3 --marker-trace
LIBS = ["-L", os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx"]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, "-o", tmp, *srcs, *LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    errs = [ln for ln in res.stderr.splitlines()
            if "packed-fp32-ops" not in ln and ln.strip() and "warning: feature" not in ln]
    if verbose and errs:
        print("\n".join(errs))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
