"""Builds the HIP library (libkda.so) in-tree for gfx950.

The library is built by one hipcc call from the kernel sources in csrc/
(kda_step.hip: decode, verify and record mode; kda_split.hip: the split
variant for small batches; kda_replay.hip: the replay; kda_probe.hip: the
page-traffic measurement aid; the headers
kda_device.hpp and kda_stages.hpp hold the shared device code, kda_host.hpp
the shared host-side checks).
Packed FP32 instructions are switched off (-packed-fp32-ops): the kernels
are written for scalar FP32 FMAs.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f)
           for f in ("kda_step.hip", "kda_split.hip", "kda_replay.hip", "kda_probe.hip")]
LIB = os.path.join(HERE, "libkda.so")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def hipcc_command(out: str = LIB) -> list:
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            f"-I{INCLUDE}", f"-I{CSRC}", "-o", out, *SOURCES]


def build_library(verbose: bool = False) -> str:
    """Compiles the csrc/ sources into libkda.so next to this file (atomically)."""
    tmp = LIB + ".tmp"
    r = subprocess.run(hipcc_command(tmp), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and r.stderr:
        print(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
