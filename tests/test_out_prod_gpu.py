"""GPU checks of the row-blocked out_prod (dq4_out_prod_rows).

llama.cpp PR "cuda: out_prod dequantizes a 2D weight in row blocks": the
weight is dequantized to F32 in row blocks of at most 256 MiB and each
block's GEMM accumulates into dst (beta 0, then 1).  The review says the new
multi-block cases (600 000 rows at 256 columns: three blocks, both src1
orientations) are the only way a wrong k-offset or a missing beta = 1 shows.

Reference: the oracle's F32 dequantization of the weight (bit-exact with the
GPU's, checked by the parity tests) times src1, summed in float64 with
numpy -- the plain definition of the sum.  Tolerance, from the arithmetic:
any FP32 summation of K products, in any order and with or without fused
multiply-adds, is within gamma_K * sum_r |B[r][i]| |W[r][j]| of the exact
sum, gamma_K = K u / (1 - K u), u = 2^-24.  The float64 reference is exact
to far below that.
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from block_wise_bit_amd import inputs
from gpu_util import check_sum_bound, out_prod_reference

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from libs import ensure_hip_library
    ensure_hip_library()


_reference = out_prod_reference
_check = check_sum_bound


@pytest.mark.parametrize("transposed", [False, True])
def test_three_blocks_600000_rows_at_256_columns(transposed):
    """The worked example of the PR: 600 000 rows at 256 columns dequantize in
    three 256 MiB F32 blocks; both src1 orientations; dst prefilled with NaN so
    that the first block's beta = 0 must overwrite it."""
    n_rows, n_cols, m = 600_000, 256, 8
    assert len(dq4.dq4_row_windows(n_rows, n_cols, 4, 256 << 20)) == 3
    x = inputs.make_inputs(n_rows * n_cols, 64, "nf4", 0.03, seed=600_000, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    rng = np.random.Generator(np.random.PCG64(1))
    b = rng.standard_normal((n_rows, m)).astype(np.float32)
    src1 = torch.from_numpy(np.ascontiguousarray(b.T) if transposed else b).cuda()
    dst = torch.full((m, n_cols), float("nan"), dtype=torch.float32, device="cuda")
    y = dq4.dq4_out_prod_rows(**dev, offset=float(x.offset), n_rows=n_rows, n_cols=n_cols,
                              blocksize=64, src1=src1, src1_transposed=transposed, dst=dst)
    exact, mag = _reference(x, n_rows, n_cols, b)
    _check(y.cpu().numpy(), exact, mag, n_rows, f"600000x256 transposed={transposed}")


def test_each_block_contributes_once():
    """B nonzero in only one row block at a time: dst equals that block's
    contribution alone, so a wrong k-offset or an accumulation into the wrong
    block shows as a large error."""
    n_rows, n_cols, m = 5000, 96, 4
    budget = 96 * 4 * 1500          # 1500 rows per block: blocks 0..3, the last 500 rows
    x = inputs.make_inputs(n_rows * n_cols, 32, "fp4", -0.02, seed=5, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    windows = dq4.dq4_row_windows(n_rows, n_cols, 4, budget)
    assert [w[1] for w in windows] == [1500, 1500, 1500, 500]
    rng = np.random.Generator(np.random.PCG64(2))
    for r0, rows in windows:
        b = np.zeros((n_rows, m), np.float32)
        b[r0:r0 + rows] = rng.standard_normal((rows, m))
        y = dq4.dq4_out_prod_rows(**dev, offset=float(x.offset), n_rows=n_rows, n_cols=n_cols,
                                  blocksize=32, src1=torch.from_numpy(b).cuda(),
                                  workspace_bytes=budget)
        exact, mag = _reference(x, n_rows, n_cols, b)
        # zero rows add exactly nothing; rows products plus the beta = 1 add
        _check(y.cpu().numpy(), exact, mag, rows + 1, f"only block at r0={r0}")


def test_output_head_shape_both_orientations():
    """The 151936 x 5376 output head in 13 F32 windows of <= 256 MiB, m = 16."""
    wl = inputs.OUTPUT_HEAD
    x = wl.inputs()
    dev = dq4.to_device(x)
    rng = np.random.Generator(np.random.PCG64(3))
    m = 16
    b = rng.standard_normal((wl.n_rows, m)).astype(np.float32)
    exact, mag = _reference(x, wl.n_rows, wl.n_cols, b)
    for transposed in (False, True):
        src1 = torch.from_numpy(np.ascontiguousarray(b.T) if transposed else b).cuda()
        y = dq4.dq4_out_prod_rows(**dev, offset=float(x.offset), n_rows=wl.n_rows,
                                  n_cols=wl.n_cols, blocksize=64, src1=src1,
                                  src1_transposed=transposed)
        _check(y.cpu().numpy(), exact, mag, wl.n_rows, f"output head transposed={transposed}")


def test_blocked_equals_whole_copy_within_bound_and_edge_cases():
    """One-row windows, odd column counts (windows off the vector path's
    alignment), a padded src1 (ld > m), the whole-copy single window, and the
    empty sum (n_rows = 0 writes zeros)."""
    n_rows, n_cols, m = 37, 101, 3
    x = inputs.make_inputs(n_rows * n_cols, 32, "nf4", 0.1, seed=37, n_rows=n_rows, n_cols=n_cols)
    dev = dq4.to_device(x)
    rng = np.random.Generator(np.random.PCG64(4))
    padded = rng.standard_normal((n_rows, m + 5)).astype(np.float32)
    src1 = torch.from_numpy(padded).cuda()[:, :m]          # ld = m + 5
    b = padded[:, :m]
    exact, mag = _reference(x, n_rows, n_cols, b)
    for budget in (n_cols * 4, n_cols * 4 * 5 + 3, n_rows * n_cols * 4):
        y = dq4.dq4_out_prod_rows(**dev, offset=float(x.offset), n_rows=n_rows, n_cols=n_cols,
                                  blocksize=32, src1=src1, workspace_bytes=budget)
        _check(y.cpu().numpy(), exact, mag, n_rows, f"budget {budget}")
    with pytest.raises(ValueError):
        dq4.dq4_out_prod_rows(**dev, offset=0.0, n_rows=n_rows, n_cols=n_cols, blocksize=32,
                              src1=src1, workspace=torch.empty(n_cols - 1, device="cuda"))
    empty = torch.empty((0, m), dtype=torch.float32, device="cuda")
    dst = torch.full((m, n_cols), 5.0, dtype=torch.float32, device="cuda")
    y = dq4.dq4_out_prod_rows(**dev, offset=0.0, n_rows=0, n_cols=n_cols, blocksize=32,
                              src1=empty, dst=dst)
    assert (y.cpu() == 0).all()
