"""The host C and C++ code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds host-only copies of the oracle (oracle/oracle.c), the task-grid
planner and decoder (csrc/sv_grid.cpp, with tests/grid_probe.cpp) and the
draft-length controller (csrc/sv_control.cpp) with
-fsanitize=address,undefined, then runs the tests that exercise them (the
oracle's pins, the task-grid checks, the controller checks) in a child
process with the ASan runtime preloaded ahead of the interpreter.  Any
out-of-bounds access, use after free or undefined behaviour (signed
overflow, misaligned access, bad shift, ...) aborts the child and fails this
test.  Leak detection is off: the interpreter itself keeps memory until exit.
No GPU code is built or run here; device code cannot be sanitised on this
hardware.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_decoding_verification_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fPIC", "-shared"]


def _asan_runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return path if path and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no host compiler")
def test_host_code_under_asan_and_ubsan(tmp_path):
    asan = _asan_runtime()
    if asan is None:
        pytest.skip("the compiler ships no ASan runtime")
    oracle_so = str(tmp_path / "liboracle_san.so")
    grid_so = str(tmp_path / "libgridprobe_san.so")
    ctl_so = str(tmp_path / "libsvcontrol_san.so")
    subprocess.check_call(["gcc", "-std=c99", *SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle_so,
                           "-lm"])
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-I", CSRC, os.path.join(CSRC, "sv_grid.cpp"),
                           os.path.join(ROOT, "tests", "grid_probe.cpp"), "-o", grid_so])
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
                           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "sv_control.cpp"), "-o", ctl_so])
    env = dict(os.environ)
    # the ASan runtime must come first among the preloaded libraries
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["ORACLE_LIB_OVERRIDE"] = oracle_so
    env["SV_GRID_PROBE_LIB"] = grid_so
    env["SV_CONTROL_LIB"] = ctl_so
    # -s: a sanitizer report goes to stderr as it happens (the child aborts)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_task_grid.py"),
           os.path.join(ROOT, "tests", "test_draft_control.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-6000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
    print(r.stdout.strip().splitlines()[-1])
