"""Helpers for the GPU parity tests: run the HIP path and the oracle on the
same host inputs and hand back raw output bits.  No arithmetic of the method
lives here -- the oracle computes, these functions only split ranges across
threads and move buffers."""
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
