"""Build the HIP library (libdq4.so) for gfx950 with hipcc, in-tree.

Flags that matter for the results:
  -ffp-contract=off          every FP32 multiply and add stays a separately
                             rounded instruction (no v_fma / v_fmac / v_mad);
  -packed-fp32-ops disabled  no packed FP32 (v_pk_*_f32) instructions;
  no -ffast-math, no -fgpu-flush-denormals-to-zero
                             IEEE round-to-nearest-even with subnormals kept.
A flag for speed only:
  -amdgpu-mfma-vgpr-form     matrix-instruction accumulators in ordinary
                             vector registers: in the direct out_prod kernels
                             the compiler otherwise shuffled accumulators
                             between accumulation registers on every step
                             (m = 32 ran 15 % slower); no other kernel changes.
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SOURCES = [os.path.join(PKG, "csrc", name)
           for name in ("dq4.hip", "dq4_unfused.hip", "dq4_gemm.hip", "dq4_out_prod_fused.hip",
                        "dq4_int8_prep.hip")]
LIBS = ["-lrocblas"]
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libdq4.so")
KERNEL_DIGESTS = os.path.join(PKG, "libdq4_kernels.json")  # written next to the library
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
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(out: str = LIBRARY, extra_flags=()) -> str:
    """Compile the library; always recompiles.  Returns the .so path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-shared", "-I", INCLUDE, "-o", tmp, *SOURCES,
           *LIBS]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    with tempfile.TemporaryDirectory() as d:
        digests = kernel_digests(device_assembly(d))
    with open(KERNEL_DIGESTS, "w") as fh:
        json.dump(digests, fh, indent=1, sort_keys=True)
    return out


def device_assembly(workdir: str) -> str:
    """gfx950 assembly of the library's kernels (for instruction checks)."""
    workdir = os.path.abspath(workdir)
    parts = []
    for src in SOURCES:
        out = os.path.join(workdir, os.path.basename(src) + "-gfx950.s")
        cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", INCLUDE, "-o", out, src]
        subprocess.run(cmd, check=True, cwd=workdir)
        with open(out) as fh:
            parts.append(fh.read())
    return "\n".join(parts)


def kernel_bodies(asm: str) -> dict:
    """{kernel symbol: its instructions, comments, directives, labels and
    s_endpgm dropped}.  A kernel's code runs to its .Lfunc_end label: the
    compiler may place blocks after an s_endpgm.  Only symbols the assembly
    declares as functions count (a device variable's label is data, not a
    kernel)."""
    functions = set(re.findall(r"^\s*\.type\s+(_Z\w+),@function", asm, flags=re.M))
    bodies = {}
    current, lines = None, []
    for line in asm.splitlines():
        if current is None:
            m = re.match(r"^(_Z\w+):", line)
            if m and m.group(1) in functions:
                current, lines = m.group(1), []
            continue
        if line.startswith(".Lfunc_end"):
            bodies[current] = "\n".join(lines)
            current = None
            continue
        code = line.split(";")[0].strip()
        if code and not code.startswith(".") and not code.endswith(":") \
                and not code.startswith("s_endpgm"):
            lines.append(code)
    return bodies


def kernel_digests(asm: str) -> dict:
    """{kernel symbol: sha256[:16] of its instructions}: identifies the exact
    code a measurement was taken on, independent of source-level edits.
    Branch labels are numbered per function in file order (.LBB<f>_<n>); the
    function number is dropped so that adding a kernel elsewhere in a file
    leaves the digests of unchanged kernels as they are."""
    return {k: hashlib.sha256(re.sub(r"\.LBB\d+_(\d+)", r".LBB_\1", v).encode()).hexdigest()[:16]
            for k, v in kernel_bodies(asm).items()}


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
