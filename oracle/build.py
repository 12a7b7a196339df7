"""Compile the C oracle with gcc (test infrastructure).

The flags matter for correctness: -ffp-contract=off keeps every FP32 multiply
and add a separately rounded IEEE operation, and neither -ffast-math nor
-march=native is used (either could fuse or reassociate float operations).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "dq4_oracle.c")
EXTRA_SOURCES = [os.path.join(HERE, "int8_prep_oracle.c")]
BUILD_DIR = os.path.join(HERE, "_build")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
          "-fPIC", "-shared"]


def library_path(build_dir: str = BUILD_DIR) -> str:
    return os.path.join(build_dir, "libdq4_oracle.so")


def build(source: str = SOURCE, build_dir: str = BUILD_DIR, extra_flags=(),
          extra_sources=None) -> str:
    """Compile `source` (and the other oracle sources) into
    build_dir/libdq4_oracle.so and return its path."""
    os.makedirs(build_dir, exist_ok=True)
    out = library_path(build_dir)
    tmp = out + ".tmp%d" % os.getpid()
    others = EXTRA_SOURCES if extra_sources is None else extra_sources
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, source, *others]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
