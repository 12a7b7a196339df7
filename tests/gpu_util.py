"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same host inputs and hand back raw output bits.  No arithmetic of the method
lives here -- the oracle computes, these functions only split ranges across
threads and move buffers (and, for the out_prod tests, sum the oracle's
weight against src1 in float64 with numpy)."""
from __future__ import annotations

import concurrent.futures
import os
import sys

import numpy as np

import block_wise_bit_amd as dq4
import oracle

_NP_BITS = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16}


def torch_dtype(dt: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def bits_of(t) -> np.ndarray:
    """Raw bits of a GPU/CPU output tensor as a numpy array."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def oracle_bits(x, dt: str, first: int = 0, count: int | None = None,
                threads: int | None = None) -> np.ndarray:
    """Oracle output for global elements [first, first+count) as raw bits."""
    count = x.n - first if count is None else count
    threads = threads or min(16, os.cpu_count() or 1)
    out = np.empty(count, dtype=np.float32 if dt == "f32" else np.uint16)
    chunk = max(1 << 20, -(-count // threads))
    chunk += (-chunk) % 8

    def one(start):
        c = min(chunk, count - start)
        out[start:start + c] = oracle.dequant_range(
            x.packed, x.scale_codes, x.nested_absmax, x.scale_codebook, x.codebook4, x.offset,
            first + start, c, x.blocksize, x.nested_blocksize, dt)

    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        list(pool.map(one, range(0, count, chunk)))
    return out.view(np.uint32) if dt == "f32" else out


def gpu_bits(x, dt: str, dev=None, out=None) -> np.ndarray:
    dev = dev or dq4.to_device(x)
    y = dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=x.blocksize,
                               nested_blocksize=x.nested_blocksize, out_dtype=torch_dtype(dt),
                               out=out)
    return bits_of(y[: x.n])


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f"{what}: {bad.size} of {want.size} elements differ; first at "
                           f"{bad[0]}: gpu {got[bad[0]]:#x} oracle {want[bad[0]]:#x}")


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


U32 = 2.0 ** -24   # unit roundoff of binary32


def out_prod_reference(x, n_rows, n_cols, b_rows_by_m, chunk_rows=16384):
    """float64 sum_r B[r][i] W[r][j] and sum_r |B[r][i]| |W[r][j]|, with W the
    oracle's F32 dequantization of the n_rows x n_cols weight x."""
    m = b_rows_by_m.shape[1]
    exact = np.zeros((m, n_cols))
    mag = np.zeros((m, n_cols))
    for r0 in range(0, n_rows, chunk_rows):
        rows = min(chunk_rows, n_rows - r0)
        w = oracle_bits(x, "f32", r0 * n_cols, rows * n_cols).view(np.float32)
        w = w.reshape(rows, n_cols).astype(np.float64)
        b = b_rows_by_m[r0:r0 + rows].astype(np.float64)
        exact += b.T @ w
        mag += np.abs(b).T @ np.abs(w)
    return exact, mag


def check_sum_bound(got, exact, mag, K, what, factor=1.0):
    """Every element within factor * gamma_K * mag of the exact sum, where
    gamma_K = K u / (1 - K u): the bound of any FP32 summation of K products,
    in any order and with or without fused multiply-adds."""
    gamma = K * U32 / (1 - K * U32)
    err = np.abs(got.astype(np.float64) - exact)
    bound = factor * gamma * mag
    worst = np.max(err / np.maximum(bound, 1e-300))
    say(f"{what}: max |err| {err.max():.3e}, worst err/bound {worst:.3e}")
    assert np.isfinite(got).all(), what
    assert (err <= bound).all(), f"{what}: error above the FP32 summation bound"
