"""Build libbef.so (HIP, gfx950) in-tree with hipcc.

    python -m bit_exact_frame_amd.build          # libbef.so
    build_host_emu(out, mutant=k)                # the tests' emulation library

The library holds the streaming row kernels (rows.hip), the ordered plan /
pair / walk kernels (walk.hip) and the host runtime behind the C ABI
(bef.cpp).  The host emulation of the kernels' steps (host_emu.cpp, test
entry points of host_emu.h) is a separate host-only library that only the
tests build and load.
Every HIP source is compiled for gfx950 with packed FP32 instructions
disabled and no floating-point contraction.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libbef.so")
ARCH = os.environ.get("BEF_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["rows.hip", "walk.hip", "bef.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops"]


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every source (always: no up-to-date check) into ``out``."""
    cmd = [HIPCC, *COMMON, *DEVICE, "-shared", "-x", "hip",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    if verbose and res.stderr:
        print(res.stderr)
    os.replace(out + ".tmp", out)
    return out


def build_host_emu(out: str, mutant: int = 0) -> str:
    """Host-only build of the emulation entry points (g++, no HIP), with an
    optional planted break in the shared step header (tests only)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", f"-DBEF_MUTANT={int(mutant)}", os.path.join(CSRC, "host_emu.cpp"),
           "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("g++ failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
