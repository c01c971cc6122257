"""Builds the plain-C programs that call libhc.so through include/hc.h.

abi_cpu: gcc, host only.  gpu_roundtrip: gcc against the HIP runtime API and the
C oracle.  Binaries land next to their sources (git-ignored)."""
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


def build_all():
    return [build("abi_cpu"), build("gpu_roundtrip")]


if __name__ == "__main__":
    for p in build_all():
        print(p)
