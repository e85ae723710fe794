"""Builds libspecverify.so in-tree for gfx950 with hipcc.

    python -m speculative_decoding_verification_amd.build

Kernels are compiled for gfx950 only, with packed-fp32 instruction selection
turned off.  The C-ABI layer is host C++ compiled by the same hipcc.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libspecverify.so")

ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument", "-I", INCLUDE,
                "-I", CSRC]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libspecverify.so (always rebuilds)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="svbuild") as tmp:
        k_obj = os.path.join(tmp, "sv_kernels.o")
        a_obj = os.path.join(tmp, "sv_api.o")
        g_obj = os.path.join(tmp, "sv_grid.o")
        c_obj = os.path.join(tmp, "sv_control.o")
        l_obj = os.path.join(tmp, "sv_lmhead.o")
        s_obj = os.path.join(tmp, "sv_sol.o")
        cmds = [
            [cc, "-x", "hip", "--offload-arch=" + ARCH, *COMMON_FLAGS, *DEVICE_FLAGS, "-c",
             os.path.join(CSRC, "sv_kernels.hip"), "-o", k_obj],
            [cc, "-x", "hip", "--offload-arch=" + ARCH, *COMMON_FLAGS, *DEVICE_FLAGS, "-c",
             os.path.join(CSRC, "sv_lmhead.hip"), "-o", l_obj],
            [cc, "-x", "hip", "--offload-arch=" + ARCH, *COMMON_FLAGS, *DEVICE_FLAGS, "-c",
             os.path.join(CSRC, "sv_sol.hip"), "-o", s_obj],
            [cc, *COMMON_FLAGS, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "sv_api.cpp"), "-o", a_obj],
            [cc, *COMMON_FLAGS, "-c", os.path.join(CSRC, "sv_grid.cpp"), "-o", g_obj],
            [cc, *COMMON_FLAGS, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "sv_control.cpp"), "-o", c_obj],
        ]
        tmp_so = os.path.join(tmp, "libspecverify.so")
        cmds.append([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", k_obj, l_obj, s_obj, a_obj, g_obj, c_obj,
                     "-o", tmp_so])
        for cmd in cmds:
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)
        shutil.copyfile(tmp_so, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
