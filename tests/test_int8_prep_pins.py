"""Pins of the LLM.int8 correction-operand oracle (CPU only).

bitsandbytes issue "Fuse LLM.int8 correction operand preparation into one
CUDA kernel", section "Exact correctness oracle": the gathered activations
are copied bit for bit, and each weight output is the FP32 product of the
int8 code and its row scale, multiplied again (a second rounding) by the
FP32 constant nearest 1/127 and converted once to FP16.  That section also
lists what the checks should reach: every int8 code, row scales of several
kinds (zero, tiny, ordinary, huge), a range of outlier counts, and column
sets in several orders, with repeats.

The oracle (oracle/int8_prep_oracle.c) is checked against
* the exact-rational IEEE model of tests/exact_ieee.py for every int8 code
  and the listed kinds of row scale;
* a binary64 closed form (exact products, one rounding per FP32 step) for
  every int8 code times 4096 row scales spread over 2^-29 .. 2^29;
* numpy fancy indexing (a library routine) for both gathers and the
  transposed layout;
* planted mistakes in a copy of its source, each of which must fail.
"""
from __future__ import annotations

import os
import shutil
import tempfile

import numpy as np
import pytest

import exact_ieee as ex
import oracle
from oracle import build as oracle_build

R127 = float(np.float32(1.0 / 127.0))   # reading: the FP32 value nearest 1/127

# zero, subnormal, normal, FP16-overflowing and the largest finite scales, plus four
# "tie-adjacent" scales: for code 1, fl32(s * R127) lands within one FP32 ulp of an
# FP16 rounding boundary, so computing s / 127 in another way (a double divide, a
# folded constant) moves the FP16 result; found by scanning all FP32 s in [64, 128)
TIE_ADJACENT = [np.uint32(v).view(np.float32).item()
                for v in (0x42FE1FC1, 0x42FE9EC1, 0x42FF1DC1, 0x42FF9CC1)]
SCB_KINDS = [0.0, 2.0 ** -149, 3 * 2.0 ** -149, 2.0 ** -126, 2.0 ** -126 * 1.5, 1e-30, 0.0078125,
             1.0, 127.0, 2.5, 1e5, 65504.0 * 127, 3.4028234663852886e38, -3.0] + TIE_ADJACENT


def _exact_subB(codes: np.ndarray, scb: np.ndarray) -> np.ndarray:
    out = np.empty((codes.size, scb.size), np.uint16)
    for j, s in enumerate(scb):
        for i, c in enumerate(codes):
            v = ex.mul32(ex.mul32(float(c), float(s)), R127)
            out[i, j] = ex.f16_bits(v)
    return out


def int8_code_domain_check(lib):
    """Every int8 code x every kind of row scale against the exact model.
    CB has one row per scale kind; cols picks every code's column."""
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    scb = np.array(SCB_KINDS, np.float32)
    N, K = scb.size, codes.size
    CB = np.tile(codes, (N, 1))
    A = np.zeros((2, K), np.uint16)
    cols = np.arange(K, dtype=np.int64)
    _, subB = oracle.int8_prep(A, CB, scb, cols, oracle=lib)
    want = _exact_subB(codes, scb)           # [code, row]
    assert np.array_equal(subB, want), "subB differs from the exact model"


def closed_form_check(lib, n_scales=4096):
    """About a million (code, row scale) pairs against the binary64 closed
    form: an int8 code times a binary32 scale is exact in binary64, as is a
    binary32 value times the binary32 constant, so each FP32 step is one
    rounding of an exact binary64 product; the FP16 step is numpy's cast."""
    rng = np.random.Generator(np.random.PCG64(17))
    scb = np.exp(rng.uniform(-20, 20, n_scales)).astype(np.float32)
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    CB = np.tile(codes, (n_scales, 1))
    _, subB = oracle.int8_prep(np.zeros((1, 256), np.uint16), CB, scb,
                               np.arange(256, dtype=np.int64), oracle=lib)
    t = (codes.astype(np.float64)[:, None] * scb.astype(np.float64)[None, :]).astype(np.float32)
    v = (t.astype(np.float64) * np.float64(np.float32(1.0 / 127.0))).astype(np.float32)
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(subB, want), "subB differs from the binary64 closed form"


def gather_check(lib, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    M, K, N = 7, 300, 11
    A = rng.integers(0, 1 << 16, size=(M, K), dtype=np.uint64).astype(np.uint16)
    CB = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    SCB = np.exp(rng.standard_normal(N)).astype(np.float32)
    for cols in (np.array([0]), np.array([K - 1]), np.array([5, 2, 5, 299, 0]),
                 np.sort(rng.choice(K, 16, replace=False)), rng.choice(K, 64, replace=True)):
        cols = cols.astype(np.int64)
        subA, subB = oracle.int8_prep(A, CB, SCB, cols, oracle=lib)
        assert np.array_equal(subA, A[:, cols]), "subA is not A[:, cols]"
        # subB is the transpose of the dequantized CB[:, cols]: row l holds column cols[l]
        for l, c in enumerate(cols):
            single = oracle.int8_prep(A[:, [c]], CB[:, [c]], SCB, np.array([0]), oracle=lib)[1][0]
            assert np.array_equal(subB[l], single), "subB row l is not column cols[l] of CB"
        assert subB.shape == (cols.size, N)


def test_int8_code_domain_exact_model():
    int8_code_domain_check(oracle.load())


def test_closed_form_million_pairs():
    closed_form_check(oracle.load())


def test_gathers_against_numpy_indexing():
    gather_check(oracle.load())


def test_examples_by_hand():
    # 127 * 1.0 * fl32(1/127) is just under 1 in FP32 and rounds to 1.0 in FP16
    A = np.zeros((1, 2), np.uint16)
    CB = np.array([[127, -128]], np.int8)
    _, subB = oracle.int8_prep(A, CB, np.array([1.0], np.float32), np.array([0, 1]))
    assert subB[0, 0] == 0x3C00                      # 1.0
    assert subB[1, 0] == 0xBC08                      # -128/127 = -1.00787... -> -1.0078125
    _, subB = oracle.int8_prep(A, CB, np.array([0.0], np.float32), np.array([1]))
    assert subB[0, 0] == 0x8000                      # -128 * +0 = -0
    with pytest.raises(ValueError):
        oracle.int8_prep(A, CB, np.array([1.0], np.float32), np.array([2]))


MUTATIONS = {
    "scale_folded": ("const float v = scaled * r127;",
                     "const float v = code * (SCB[n] * r127); (void)scaled;"),
    "divide_in_double": ("const float v = scaled * r127;",
                         "const float v = (float)((double)scaled / 127.0); (void)r127;"),
    "not_transposed": ("subB[l * N + n] = dq4o_f32_to_f16(v);",
                       "subB[n * L + l] = dq4o_f32_to_f16(v);"),
    "activation_not_gathered": ("subA[r * L + l] = A[r * K + cols[l]];",
                                "subA[r * L + l] = A[r * K + l];"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    d = tempfile.mkdtemp(prefix="int8_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(name, mutant_dir):
    old, new = MUTATIONS[name]
    src = open(oracle_build.EXTRA_SOURCES[0]).read()
    assert src.count(old) == 1
    path = os.path.join(mutant_dir, name)
    os.makedirs(path, exist_ok=True)
    cfile = os.path.join(path, "int8_prep_oracle.c")
    with open(cfile, "w") as fh:
        fh.write(src.replace(old, new))
    oracle_build.build(oracle_build.SOURCE, path, extra_sources=[cfile])
    lib = oracle.load(oracle_build.library_path(path))
    failed = 0
    for check in (int8_code_domain_check, closed_form_check, gather_check):
        try:
            check(lib)
        except AssertionError:
            failed += 1
    assert failed > 0, f"planted mistake {name} passed every pin"
