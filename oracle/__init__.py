"""CPU oracle for nested block-wise 4-bit dequantization (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and the oracle never
imports the product path.

The arithmetic lives in ``dq4_oracle.c``: a plain single-threaded C
transcription of the three-step nested dequantization described in the
bitsandbytes issue "Fuse nested scale reconstruction into SM103 4-bit
dequantization" (sections "Problem", "Proposed experiment" and "Correctness
requirements"), compiled with ``gcc -O2 -ffp-contract=off``.  This module only
marshals numpy arrays into it.

Pins (what the oracle is checked against, in ``tests/test_oracle_pins.py``):
  * the FP16/BF16 conversions: every one of the 2^32 binary32 inputs against
    torch's CPU conversions, and a large subset against numpy's FP16 cast;
  * scale reconstruction and value decode: an exact-rational model of IEEE
    round-to-nearest-even arithmetic, brute force over every scale code and
    every 4-bit code in both nibble positions, several nested groups, both
    offset signs, NF4- and FP4-style tables and all three output types;
  * tails, partial outer blocks and partial nested groups for every block
    size from 32 to 4096;
  * the special case scale = 1 (a plain table decode) and the decode-back
    invariant out / scale -> codebook entry;
  * rows per block against the worked example of the llama.cpp PR
    (600 000 rows at 256 columns -> three blocks) and the output-head window
    plan (151 936 x 5 376 -> 12 483 rows per block, 13 windows);
  * mutation checks: planted mistakes in a copy of the C source (contracted
    multiply-add, swapped nibble order, dropped offset, wrong group index)
    must each fail a pin.
Parity unpinned: the upstream library's own NF4/FP4 tables and nibble order
(the pages print neither; the tables are inputs here) and NaN payloads.

``int8_prep_oracle.c`` is the oracle of the LLM.int8 correction-operand
preparation (bitsandbytes issue "Fuse LLM.int8 correction operand preparation
into one CUDA kernel"), pinned in ``tests/test_int8_prep_pins.py`` against
the exact-rational model over the whole int8 code domain and zero, normal,
subnormal-adjacent and large finite row scales, and against numpy indexing for
the gathers.  Parity unpinned: the digits of the upstream reciprocal-127
constant (read as the FP32 value nearest 1/127).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import library_path, build as _build

F32, F16, BF16 = 0, 1, 2
_DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
_NP_OUT = {F32: np.float32, F16: np.uint16, BF16: np.uint16}


class OracleLib:
    """ctypes handle on one compiled copy of the C oracle."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        lib.dq4o_dequant_range.argtypes = [P, P, P, P, P, f32, i64, i64, i32, i32, i32, P]
        lib.dq4o_dequant_range.restype = ctypes.c_int
        lib.dq4o_dequant_rows.argtypes = [P, P, P, P, P, f32, i64, i64, i64, i64, i32, i32,
                                          i32, P]
        lib.dq4o_dequant_rows.restype = ctypes.c_int
        lib.dq4o_rows_per_block.argtypes = [i64, i64, i64]
        lib.dq4o_rows_per_block.restype = i64
        lib.dq4o_f32_to_f16_array.argtypes = [P, P, i64]
        lib.dq4o_f32_to_f16_array.restype = None
        lib.dq4o_f32_to_bf16_array.argtypes = [P, P, i64]
        lib.dq4o_f32_to_bf16_array.restype = None
        lib.dq4o_int8_prep.argtypes = [P, i64, i64, P, P, i64, P, i64, P, P]
        lib.dq4o_int8_prep.restype = ctypes.c_int
        self.path = path
        self.lib = lib


_default = None


def load(path: str | None = None) -> OracleLib:
    """The oracle built from dq4_oracle.c (compiled on first use), or the copy at `path`."""
    global _default
    if path is not None:
        return OracleLib(path)
    if _default is None:
        p = library_path()
        if not os.path.exists(p):
            _build()
        _default = OracleLib(p)
    return _default


def _dtype_code(out_dtype) -> int:
    if isinstance(out_dtype, str):
        return _DTYPES[out_dtype]
    return int(out_dtype)


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check_sizes(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                 end, blocksize, nested_blocksize):
    if end > 0:
        nb = -(-end // blocksize)
        ng = -(-nb // nested_blocksize)
        assert packed.size >= -(-end // 2), "packed too short"
        assert scale_codes.size >= nb, "scale_codes too short"
        assert nested_absmax.size >= ng, "nested_absmax too short"
    assert scale_codebook.size == 256 and codebook4.size == 16


def dequant_range(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                  offset, first, count, blocksize, nested_blocksize=256,
                  out_dtype="f16", oracle: OracleLib | None = None) -> np.ndarray:
    """Elements [first, first+count) of the flat tensor; F32 as float32, F16/BF16 as uint16 bits."""
    lib = (oracle or load()).lib
    dt = _dtype_code(out_dtype)
    packed = _c(packed, np.uint8)
    scale_codes = _c(scale_codes, np.uint8)
    nested_absmax = _c(nested_absmax, np.float32)
    scale_codebook = _c(scale_codebook, np.float32)
    codebook4 = _c(codebook4, np.float32)
    _check_sizes(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                 first + count, blocksize, nested_blocksize)
    out = np.empty(count, dtype=_NP_OUT[dt])
    rc = lib.dq4o_dequant_range(_ptr(packed), _ptr(scale_codes), _ptr(nested_absmax),
                                _ptr(scale_codebook), _ptr(codebook4),
                                ctypes.c_float(np.float32(offset)), first, count,
                                blocksize, nested_blocksize, dt, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def dequant(packed, scale_codes, nested_absmax, scale_codebook, codebook4, offset,
            n, blocksize, nested_blocksize=256, out_dtype="f16",
            oracle: OracleLib | None = None) -> np.ndarray:
    """The whole flat tensor of n elements."""
    return dequant_range(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                         offset, 0, n, blocksize, nested_blocksize, out_dtype, oracle)


def dequant_rows(packed, scale_codes, nested_absmax, scale_codebook, codebook4, offset,
                 n_rows, n_cols, r0, rows, blocksize, nested_blocksize=256,
                 out_dtype="f16", oracle: OracleLib | None = None) -> np.ndarray:
    """Rows [r0, r0+rows) of an n_rows x n_cols weight, as rows*n_cols elements."""
    lib = (oracle or load()).lib
    dt = _dtype_code(out_dtype)
    if not (0 <= r0 and 0 <= rows and r0 + rows <= n_rows):
        raise ValueError("row window out of range")
    packed = _c(packed, np.uint8)
    scale_codes = _c(scale_codes, np.uint8)
    nested_absmax = _c(nested_absmax, np.float32)
    scale_codebook = _c(scale_codebook, np.float32)
    codebook4 = _c(codebook4, np.float32)
    _check_sizes(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                 (r0 + rows) * n_cols, blocksize, nested_blocksize)
    out = np.empty(rows * n_cols, dtype=_NP_OUT[dt])
    rc = lib.dq4o_dequant_rows(_ptr(packed), _ptr(scale_codes), _ptr(nested_absmax),
                               _ptr(scale_codebook), _ptr(codebook4),
                               ctypes.c_float(np.float32(offset)), n_rows, n_cols, r0, rows,
                               blocksize, nested_blocksize, dt, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def rows_per_block(n_cols: int, elem_bytes: int, budget_bytes: int,
                   oracle: OracleLib | None = None) -> int:
    return int((oracle or load()).lib.dq4o_rows_per_block(n_cols, elem_bytes, budget_bytes))


def f32_to_f16_bits(bits_u32: np.ndarray, oracle: OracleLib | None = None) -> np.ndarray:
    """binary32 bit patterns -> IEEE binary16 bit patterns (round to nearest even)."""
    lib = (oracle or load()).lib
    a = _c(bits_u32, np.uint32)
    out = np.empty(a.size, dtype=np.uint16)
    lib.dq4o_f32_to_f16_array(_ptr(a), _ptr(out), a.size)
    return out


def f32_to_bf16_bits(bits_u32: np.ndarray, oracle: OracleLib | None = None) -> np.ndarray:
    """binary32 bit patterns -> bfloat16 bit patterns (round to nearest even)."""
    lib = (oracle or load()).lib
    a = _c(bits_u32, np.uint32)
    out = np.empty(a.size, dtype=np.uint16)
    lib.dq4o_f32_to_bf16_array(_ptr(a), _ptr(out), a.size)
    return out


def int8_prep(A_bits: np.ndarray, CB: np.ndarray, SCB: np.ndarray, cols: np.ndarray,
              oracle: OracleLib | None = None):
    """LLM.int8 correction operands: subA (M x L, A's raw 16-bit values) and
    subB (L x N, FP16 bits) -- see int8_prep_oracle.c."""
    lib = (oracle or load()).lib
    A_bits = _c(A_bits, np.uint16)
    CB = _c(CB, np.int8)
    SCB = _c(SCB, np.float32)
    cols = _c(cols, np.int64)
    M, K = A_bits.shape
    N = CB.shape[0]
    assert CB.shape == (N, K) and SCB.shape == (N,)
    L = cols.size
    subA = np.empty((M, L), np.uint16)
    subB = np.empty((L, N), np.uint16)
    rc = lib.dq4o_int8_prep(_ptr(A_bits), M, K, _ptr(CB), _ptr(SCB), N, _ptr(cols), L,
                            _ptr(subA), _ptr(subB))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return subA, subB
