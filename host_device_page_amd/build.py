"""Builds libhc.so (HIP kernels + C ABI) for gfx950 with hipcc, in the package directory.

    python -m host_device_page_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhc.so")
SOURCES = ["hc_api.cpp", "hc_layout.cpp", "hc_plan.cpp", "hc_loader.cpp", "hc_h2h.cpp", "hc_kernels.hip", "hc_exchange.hip", "hc_noalloc.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))

# Packed fp32 instructions are kept out of every code object (the copy kernels
# have no float arithmetic; the flag makes sure none is generated).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC]


# roctx ranges around the entry points (rocprofiler-sdk's marker library)
LIBS = ["-L" + os.path.join(ROCM, "lib"), "-lrocprofiler-sdk-roctx"]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile libhc.so; `defines` are extra -D tuning knobs (e.g. HC_UNROLL=16)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-o", tmp, *srcs, *LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "unknown target feature", "warning: argument unused")
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if ln.strip() and not any(x in ln for x in noise)]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
