"""The C ABI used from plain C programs (no Python, no torch)."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c"))
import build as cbuild  # noqa: E402


def test_c_program_without_gpu():
    exe = cbuild.build("abi_cpu")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert "abi_cpu ok" in r.stdout


@pytest.mark.gpu
def test_c_program_round_trip_on_gpu():
    exe = os.path.join(HERE, "c", "gpu_roundtrip")
    assert os.path.exists(exe), "build it with __graft_entry__.build() (tests/c/build.py)"
    print("[c] gpu_roundtrip", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu_roundtrip ok" in r.stdout
