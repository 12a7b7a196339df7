"""Build the HIP library (libdq4.so) for gfx950 with hipcc, in-tree.

Flags that matter for the results:
  -ffp-contract=off          every FP32 multiply and add stays a separately
                             rounded instruction (no v_fma / v_fmac / v_mad);
  -packed-fp32-ops disabled  no packed FP32 (v_pk_*_f32) instructions;
  no -ffast-math, no -fgpu-flush-denormals-to-zero
                             IEEE round-to-nearest-even with subnormals kept.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCE = os.path.join(PKG, "csrc", "dq4.hip")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libdq4.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fPIC",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIBRARY, extra_flags=()) -> str:
    """Compile the library; always recompiles.  Returns the .so path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-shared", "-I", INCLUDE, "-o", tmp, SOURCE]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def device_assembly(workdir: str) -> str:
    """gfx950 assembly of the library's kernels (for instruction checks)."""
    workdir = os.path.abspath(workdir)
    cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", INCLUDE,
           "-o", os.path.join(workdir, "dq4-gfx950.s"), SOURCE]
    subprocess.run(cmd, check=True, cwd=workdir)
    with open(os.path.join(workdir, "dq4-gfx950.s")) as fh:
        return fh.read()


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
