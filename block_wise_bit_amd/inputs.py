"""Seeded synthetic inputs for nested 4-bit dequantization.

This module only draws random numbers and lays them out; it holds none of the
dequantization arithmetic.  Both the HIP path (tests, bench, smoke) and the
CPU oracle consume the buffers it makes.

The pages measure on "representative weights" of given shapes (bitsandbytes
issue "Fuse nested scale reconstruction into SM103 4-bit dequantization",
section "B300 evidence plan") and publish no data; these synthetic inputs
stand in for them:

* packed 4-bit values and uint8 scale codes: iid uniform over 0..255;
* nested absmax: lognormal(mu=-3, sigma=0.5), rounded once to FP32;
* scale codebook: 256 iid uniform values in [-1, 1), sorted ascending;
* NF4-style codebook: 15 iid uniform values in [-1, 1) plus an exact 0.0,
  sorted ascending;
* FP4-style codebook: the 16 E2M1 code points (sign-magnitude, bit 3 the
  sign, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) divided by 6 so the largest
  magnitude is 1; it holds -0.0 and is not sorted.  The pages name FP4 but
  print no table, so this table is a reading, and the kernels are
  table-driven either way.

Random numbers come from numpy's PCG64 generator seeded per workload, so a
(workload, seed) pair always yields the same bytes on any machine with the
same numpy.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np

NESTED_BLOCKSIZE = 256

_E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


@dataclasses.dataclass
class NestedInputs:
    """Host buffers of one nested-quantized tensor of n elements."""

    packed: np.ndarray          # uint8, ceil(n/2): element 2j in the low nibble of byte j
    scale_codes: np.ndarray     # uint8, ceil(n/blocksize)
    nested_absmax: np.ndarray   # float32, ceil(n_blocks/256)
    scale_codebook: np.ndarray  # float32, 256
    codebook4: np.ndarray       # float32, 16
    offset: np.float32
    n: int
    blocksize: int
    nested_blocksize: int = NESTED_BLOCKSIZE
    fmt: str = "nf4"
    n_rows: Optional[int] = None
    n_cols: Optional[int] = None
    seed: int = 0

    @property
    def n_blocks(self) -> int:
        return -(-self.n // self.blocksize)

    @property
    def n_groups(self) -> int:
        return -(-self.n_blocks // self.nested_blocksize)

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.packed, self.scale_codes, self.nested_absmax, self.scale_codebook,
                  self.codebook4, np.array([self.offset], np.float32)):
            h.update(np.ascontiguousarray(a).tobytes())
        return h.hexdigest()[:16]


def nf4_style_codebook(rng: np.random.Generator) -> np.ndarray:
    vals = np.concatenate([_uniform_pm1(rng, 15), np.zeros(1, np.float32)])
    return np.sort(vals).astype(np.float32)


def fp4_style_codebook() -> np.ndarray:
    table = np.empty(16, np.float32)
    for code in range(16):
        mag = np.float32(_E2M1_MAGNITUDES[code & 7]) / np.float32(6.0)
        table[code] = -mag if code & 8 else mag
    return table


def _uniform_pm1(rng: np.random.Generator, size: int) -> np.ndarray:
    # 24-bit uniform u in [0, 1) on the 2^-24 grid, mapped to 2u - 1 exactly in FP32
    u = rng.integers(0, 1 << 24, size=size, dtype=np.int64).astype(np.float64) / float(1 << 24)
    return (2.0 * u - 1.0).astype(np.float32)


def make_inputs(n: int, blocksize: int, fmt: str = "nf4", offset: float = 0.03,
                seed: int = 0, nested_blocksize: int = NESTED_BLOCKSIZE,
                n_rows: Optional[int] = None, n_cols: Optional[int] = None) -> NestedInputs:
    """Random inputs of the pages' workload shape and distributions."""
    if n_rows is not None:
        assert n_cols is not None and n_rows * n_cols == n
    rng = np.random.Generator(np.random.PCG64(seed))
    n_bytes = (n + 1) // 2
    nb = -(-n // blocksize) if n else 0
    ng = -(-nb // nested_blocksize) if nb else 0
    packed = np.frombuffer(rng.bytes(n_bytes), dtype=np.uint8).copy()
    scale_codes = np.frombuffer(rng.bytes(nb), dtype=np.uint8).copy()
    nested_absmax = np.exp(-3.0 + 0.5 * rng.standard_normal(ng)).astype(np.float32)
    scale_codebook = np.sort(_uniform_pm1(rng, 256)).astype(np.float32)
    if fmt == "nf4":
        codebook4 = nf4_style_codebook(rng)
    elif fmt == "fp4":
        codebook4 = fp4_style_codebook()
    else:
        raise ValueError("fmt must be 'nf4' or 'fp4'")
    return NestedInputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                        np.float32(offset), n, blocksize, nested_blocksize, fmt,
                        n_rows, n_cols, seed)


# ----------------------------------------------------------------------------
# Named workloads: the shapes of the pages' primary standalone matrix, the
# odd-tail / block-size sweep, and the output-head row-window case.
# ----------------------------------------------------------------------------
SEED_BASE = 0x5EED0000


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_rows: int
    n_cols: int
    blocksize: int
    fmt: str
    out_dtype: str
    offset: float
    seed: int

    @property
    def n(self) -> int:
        return self.n_rows * self.n_cols

    def inputs(self) -> NestedInputs:
        return make_inputs(self.n, self.blocksize, self.fmt, self.offset, self.seed,
                           n_rows=self.n_rows, n_cols=self.n_cols)


def _wl(name, rows, cols, bs, fmt, dt, off, idx):
    return Workload(name, rows, cols, bs, fmt, dt, off, SEED_BASE + idx)


# 4096 x 4096 NF4 -> FP32, offset +0.03
SQUARE_4096_F32 = _wl("nf4_f32_4096x4096_bs64", 4096, 4096, 64, "nf4", "f32", 0.03, 1)
# 28672 x 8192 NF4 -> FP16, offset +0.03: the headline bandwidth case
HEADLINE = _wl("nf4_f16_28672x8192_bs64", 28672, 8192, 64, "nf4", "f16", 0.03, 3)
# 151936 x 5376 NF4 output head, dequantized in <= 256 MiB FP32 row windows
OUTPUT_HEAD = _wl("nf4_f32_rows_151936x5376_bs64", 151936, 5376, 64, "nf4", "f32", 0.03, 5)
# odd 1-D length for the block-size / tail sweep
TAIL_SWEEP_N = 4096 * 11008 + 37
TAIL_SWEEP_BLOCKSIZES = (32, 64, 128, 256, 512, 1024, 2048, 4096)
TAIL_SWEEP_OFFSETS = (-0.1, 0.0, 0.1)


def mid_matrix_workloads():
    """{FP4, NF4} x {11008x4096, 4096x11008} x {FP16, BF16, FP32}, bs 64, offset -0.02."""
    out = []
    for fmt in ("nf4", "fp4"):
        for rows, cols in ((11008, 4096), (4096, 11008)):
            for dt in ("f16", "bf16", "f32"):
                out.append(_wl(f"{fmt}_{dt}_{rows}x{cols}_bs64", rows, cols, 64, fmt, dt,
                               -0.02, 2))
    return out


def tail_sweep_workloads():
    """1-D n = 4096*11008+37, every block size 32..4096, NF4/FP4, FP16, offsets -0.1/0/+0.1."""
    out = []
    for bs in TAIL_SWEEP_BLOCKSIZES:
        for fmt in ("nf4", "fp4"):
            for off in TAIL_SWEEP_OFFSETS:
                out.append(_wl(f"{fmt}_f16_tail_bs{bs}_off{off:+.1f}", 1, TAIL_SWEEP_N, bs, fmt,
                               "f16", off, 4))
    return out
