"""GPU checks of the row-blocked out_prod (dq4_out_prod_rows).

llama.cpp PR "cuda: out_prod dequantizes a 2D weight in row blocks": the
weight is dequantized to F32 in row blocks of at most 256 MiB and each
block's GEMM accumulates into dst (beta 0, then 1).  The review says the new
multi-block cases (600 000 rows at 256 columns: three blocks, both src1
orientations) are the only way a wrong k-offset or a missing beta = 1 shows.

Two kinds of check at the PR's sizes (600 000 x 256, three row blocks) and
the output head's (151 936 x 5 376, 13 row blocks), both src1 orientations:
* selection-matrix src1 (one 1 per column, on rows chosen so that every row
  block, its first and last row, is hit): dst must equal the oracle's weight
  rows exactly, so a wrong k-offset, a dropped block or a missing beta = 1
  fails outright;
* random src1 against the oracle's F32 weight times src1 summed in float64
  (the plain definition of the sum), within the FP32 summation bound of
  tests/sum_bounds.py; tests/test_sum_bounds.py shows on the CPU that on these
  very inputs a dst missing any one row block fails that bound.
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from block_wise_bit_amd import inputs
import out_prod_cases as cases
from gpu_util import check_selection_route, check_sum_bound, out_prod_reference

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


def _route(dev, x, n_rows, n_cols):
    def call(**kw):
        return dq4.dq4_out_prod_rows(**dev, offset=float(x.offset), n_rows=n_rows,
                                     n_cols=n_cols, blocksize=64, **kw)
    return call


@pytest.mark.parametrize("transposed", [False, True])
def test_three_blocks_600000_rows_at_256_columns(transposed):
    """The worked example of the PR: 600 000 rows at 256 columns dequantize in
    three 256 MiB F32 blocks; both src1 orientations; dst prefilled with NaN so
    that the first block's beta = 0 must overwrite it."""
    case = cases.PR_EXAMPLE
    n_rows, n_cols = case["n_rows"], case["n_cols"]
    assert len(dq4.dq4_row_windows(n_rows, n_cols, 4, 256 << 20)) == 3
    x = cases.pr_example_weight()
    dev = dq4.to_device(x)
    b = cases.random_src1(case)
    src1 = torch.from_numpy(np.ascontiguousarray(b.T) if transposed else b).cuda()
    dst = torch.full((case["m"], n_cols), float("nan"), dtype=torch.float32, device="cuda")
    y = _route(dev, x, n_rows, n_cols)(src1=src1, src1_transposed=transposed, dst=dst)
    exact, mag = _reference(x, n_rows, n_cols, b)
    _check(y.cpu().numpy(), exact, mag, n_rows, f"600000x256 transposed={transposed}")


@pytest.mark.parametrize("m", [8, 128])
@pytest.mark.parametrize("transposed", [False, True])
def test_selection_600000_rows_at_256_columns_is_bit_exact(m, transposed):
    """Selection-matrix src1 at the PR's size: every row block (and both rows
    at each block edge) is selected; dst equals the weight rows exactly."""
    case = cases.PR_EXAMPLE
    n_rows, n_cols = case["n_rows"], case["n_cols"]
    x = cases.pr_example_weight()
    dev = dq4.to_device(x)
    windows = cases.row_windows(n_rows, n_cols)
    groups = cases.selection_groups(cases.target_rows(n_rows, windows), m)
    check_selection_route(_route(dev, x, n_rows, n_cols), x, n_rows, n_cols, groups,
                          transposed, f"blocked 600000x256 m={m} transposed={transposed}")


@pytest.mark.parametrize("m", [16, 512])
def test_selection_output_head_is_bit_exact(m):
    """Selection-matrix src1 over the 151 936 x 5 376 output head's 13 row
    blocks, both orientations: dst equals the weight rows exactly."""
    wl = inputs.OUTPUT_HEAD
    x = cases.output_head_weight()
    dev = dq4.to_device(x)
    windows = cases.row_windows(wl.n_rows, wl.n_cols)
    assert len(windows) == 13
    groups = cases.selection_groups(cases.target_rows(wl.n_rows, windows), m)
    for transposed in (False, True):
        check_selection_route(_route(dev, x, wl.n_rows, wl.n_cols), x, wl.n_rows, wl.n_cols,
                              groups, transposed, f"blocked output head m={m} "
                                                  f"transposed={transposed}")


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
    case = cases.OUTPUT_HEAD
    n_rows, n_cols = case["n_rows"], case["n_cols"]
    x = cases.output_head_weight()
    dev = dq4.to_device(x)
    b = cases.random_src1(case)
    exact, mag = _reference(x, n_rows, n_cols, b)
    for transposed in (False, True):
        src1 = torch.from_numpy(np.ascontiguousarray(b.T) if transposed else b).cuda()
        y = _route(dev, x, n_rows, n_cols)(src1=src1, src1_transposed=transposed)
        _check(y.cpu().numpy(), exact, mag, n_rows, f"output head transposed={transposed}")


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
