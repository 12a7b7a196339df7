"""Sanitizer runs on host code (CPU only).

* The oracle, built with gcc -fsanitize=address,undefined, runs edge cases on
  heap buffers of exactly the defined sizes (tests/sanitize/oracle_driver.c):
  any read past the last packed byte, code or absmax is reported.
* The C ABI's host-side validation, built with AddressSanitizer and UBSan on
  the host code only (each -fsanitize= behind -Xarch_host; the GPU code is
  built as usual), runs every rejected or no-op call
  (tests/sanitize/abi_driver.cpp).  None of these calls reaches the GPU.
"""
import os
import subprocess

import pytest

from block_wise_bit_amd import build as dq4_build
from oracle import build as oracle_build

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = os.path.join(HERE, "sanitize")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
          os.path.join(SAN, "oracle_driver.c"), oracle_build.SOURCE, *oracle_build.EXTRA_SOURCES])
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0"))
    assert "0 failures" in r.stdout


def test_abi_validation_under_host_asan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    _run([dq4_build.hipcc(), *dq4_build.HIPCC_FLAGS, *host_san, "-g", "-I", dq4_build.INCLUDE,
          "-o", exe, os.path.join(SAN, "abi_driver.cpp"), *dq4_build.SOURCES, *dq4_build.LIBS])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:protect_shadow_gap=0")
    r = _run([exe], env=env)
    assert "0 failures" in r.stdout


def test_planted_overread_is_reported(tmp_path):
    """Control: a copy of the oracle that reads the packed byte of element
    i + 1 instead of i must be caught by the exact-size buffers."""
    src = open(oracle_build.SOURCE).read()
    old = "const uint8_t byte = packed[i / 2];"
    assert src.count(old) == 1
    bad = tmp_path / "dq4_oracle_overread.c"
    bad.write_text(src.replace(old, "const uint8_t byte = packed[(i + 1) / 2];"))
    exe = str(tmp_path / "oracle_driver_bad")
    _run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-o", exe, os.path.join(SAN, "oracle_driver.c"), str(bad),
          *oracle_build.EXTRA_SOURCES])
    r = subprocess.run([exe], capture_output=True, text=True,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr
