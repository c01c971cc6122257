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


@pytest.mark.parametrize("kind,banner", [("tsan", "sanitizer: thread"), ("asan", "sanitizer: address")])
def test_host_machinery_under_sanitizers(kind, banner):
    """The loader thread and the host-to-host worker pool, stressed from several threads,
    under ThreadSanitizer and under AddressSanitizer + UndefinedBehaviorSanitizer."""
    exe = cbuild.build_sanitized(kind)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 second_deadlock_stack=1",
               ASAN_OPTIONS="detect_leaks=1 abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1 print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = "\n".join(ln for ln in r.stderr.splitlines() if "burst enqueue failed" not in ln)
    assert r.returncode == 0, report[-4000:]
    assert banner in r.stdout and "sanitize_host ok" in r.stdout
    assert "WARNING: ThreadSanitizer" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr


def test_write_back_planner_under_sanitizers():
    """The staged write-back planner, executed on host buffers by a model of the device
    side for 1200 random lists, layouts and chunk sizes, under ASan + UBSan."""
    exe = cbuild.build_sanitized("asan", "plan_host")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="halt_on_error=1 print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "plan_host ok" in r.stdout and "runtime error" not in r.stderr


@pytest.mark.gpu
def test_c_program_round_trip_on_gpu():
    exe = os.path.join(HERE, "c", "gpu_roundtrip")
    assert os.path.exists(exe), "build it with __graft_entry__.build() (tests/c/build.py)"
    print("[c] gpu_roundtrip", flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu_roundtrip ok" in r.stdout
