"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same host inputs and hand back raw output bits.  No arithmetic of the method
lives here -- the oracle computes, these functions only split ranges across
threads and move buffers (and, for the out_prod tests, sum the oracle's
weight against src1 in float64 with numpy; the FP32 summation bounds those
sums are checked with live in sum_bounds.py)."""
from __future__ import annotations

import concurrent.futures
import os
import sys

import numpy as np

import block_wise_bit_amd as dq4
import oracle
from sum_bounds import U32, check_sum_bound  # noqa: F401  (re-exported for the GPU tests)

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


def out_prod_reference(x, n_rows, n_cols, b_rows_by_m, chunk_rows=16384):
    """float64 sum_r B[r][i] W[r][j] and sum_r |B[r][i]| |W[r][j]|, with W the
    oracle's F32 dequantization of the n_rows x n_cols weight x."""
    parts, mag = out_prod_reference_parts(
        x, n_cols, b_rows_by_m,
        [(r0, min(chunk_rows, n_rows - r0)) for r0 in range(0, n_rows, chunk_rows)])
    return sum(parts, np.zeros_like(mag)), mag


def out_prod_reference_parts(x, n_cols, b_rows_by_m, row_ranges, chunk_rows=16384):
    """For each (r0, rows) of row_ranges, the float64 contribution
    sum_{r in [r0, r0+rows)} B[r][i] W[r][j]; and sum_r |B[r][i]| |W[r][j]|
    over the union of the ranges.  W is the oracle's F32 dequantization."""
    m = b_rows_by_m.shape[1]
    mag = np.zeros((m, n_cols))
    parts = []
    for r0, rows in row_ranges:
        part = np.zeros((m, n_cols))
        for c0 in range(r0, r0 + rows, chunk_rows):
            c = min(chunk_rows, r0 + rows - c0)
            w = oracle_bits(x, "f32", c0 * n_cols, c * n_cols).view(np.float32)
            w = w.reshape(c, n_cols).astype(np.float64)
            b = b_rows_by_m[c0:c0 + c].astype(np.float64)
            part += b.T @ w
            mag += np.abs(b).T @ np.abs(w)
        parts.append(part)
    return parts, mag


def weight_rows(x, n_cols, rows) -> np.ndarray:
    """The oracle's F32 weight rows `rows` (any order, repeats allowed), as a
    len(rows) x n_cols float32 array."""
    out = np.empty((len(rows), n_cols), np.float32)
    for k, r in enumerate(rows):
        out[k] = oracle_bits(x, "f32", int(r) * n_cols, n_cols, threads=1).view(np.float32)
    return out


def check_selection_route(route, x, n_rows, n_cols, groups, transposed, what):
    """Full-size bit check of an out_prod route with selection-matrix src1:
    for each group `sel` of weight rows, src1 has B[sel[i]][i] = 1 and zeros
    elsewhere, so dst row i is one exact product 1 * W[sel[i]][j] plus exact
    zeros -- in any summation order, row block or row split -- and must equal
    the oracle's weight row sel[i].  dst starts as NaN, so the first row
    block's beta = 0 must overwrite it.  Values are compared (-0.0 == +0.0:
    a zero product may carry either sign into the sum)."""
    import torch
    from out_prod_cases import selection_src1
    for g, sel in enumerate(groups):
        b = selection_src1(n_rows, sel)
        src1 = torch.from_numpy(np.ascontiguousarray(b.T) if transposed else b).cuda()
        dst = torch.full((len(sel), n_cols), float("nan"), dtype=torch.float32, device="cuda")
        y = route(src1=src1, src1_transposed=transposed, dst=dst).cpu().numpy()
        want = weight_rows(x, n_cols, sel)
        bad = np.argwhere(~(y == want))
        assert bad.size == 0, (f"{what} group {g}: {bad.shape[0]} mismatches, first at (i, j) = "
                               f"{tuple(bad[0])}, weight row {sel[bad[0][0]]}: "
                               f"{y[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}")
    say(f"{what}: {len(groups)} selection calls bit-exact")
