"""Builds the plain-C programs that call libhc.so through include/hc.h.

abi_cpu: gcc, host only.  gpu_roundtrip: gcc against the HIP runtime API and the
C oracle.  sanitize_host_{tsan,asan}: the loader and host-to-host sources built under
a sanitizer; plan_host_asan: the write-back planner under ASan + UBSan (host code
only).  Binaries land next to their sources
(git-ignored)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "host_device_page_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM = "/opt/rocm"


def build(name: str) -> str:
    src = os.path.join(HERE, name + ".c")
    out = os.path.join(HERE, name)
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), "-I", ORACLE,
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), src, "-o", out,
           "-L", PKG, "-lhc", f"-Wl,-rpath,{PKG}", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    if name == "gpu_roundtrip":
        cmd += ["-L", ORACLE, "-lorc", f"-Wl,-rpath,{ORACLE}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {name} failed:\n{r.stderr}")
    return out


# Host-only builds of the CPU-side machinery (loader thread, host-to-host workers)
# under a sanitizer; g++ only, no GPU code in them.
SANITIZERS = {
    "tsan": ["-fsanitize=thread"],
    "asan": ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"],
}
HOST_SOURCES = {"sanitize_host": ["hc_loader.cpp", "hc_h2h.cpp", "hc_layout.cpp"],
                "plan_host": ["hc_plan.cpp", "hc_layout.cpp"]}


# ThreadSanitizer comes from ROCm's clang: its runtime intercepts pthread_cond_clockwait,
# which libstdc++ uses for timed waits and which the system gcc's libtsan does not see
# (every timed wait would then read as a lock that was never released).
COMPILERS = {"tsan": os.path.join(ROCM, "llvm", "bin", "clang++"), "asan": "g++"}


def build_sanitized(kind: str, program: str = "sanitize_host") -> str:
    out = os.path.join(HERE, f"{program}_{kind}")
    csrc = os.path.join(PKG, "csrc")
    cmd = [COMPILERS[kind], "-std=c++17", "-g", "-O1", "-pthread", "-Wall", *SANITIZERS[kind],
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           "-I", os.path.join(ROCM, "include"), os.path.join(HERE, program + ".cpp"),
           *[os.path.join(csrc, s) for s in HOST_SOURCES[program]], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building {program} ({kind}) failed:\n{r.stderr}")
    return out


def build_all():
    return [build("abi_cpu"), build("gpu_roundtrip")]


if __name__ == "__main__":
    for p in build_all():
        print(p)
