"""Negative controls, on the CPU, for the FP32 summation bound that the
random-src1 out_prod checks use (tests/test_out_prod_gpu.py and
tests/test_out_prod_fused_gpu.py), on exactly those checks' inputs.

llama.cpp PR "cuda: out_prod dequantizes a 2D weight in row blocks" (section
"Measured" and the approving review): only the multi-block sizes -- 600 000
rows at 256 columns in three row blocks, and here also the 151 936 x 5 376
output head in 13 -- show a wrong k-offset or a missing beta = 1.  A check at
those sizes is worth something only if a dst that drops one row block, or one
row split of the fused route, fails it.  The deterministic bound gamma_K does
not (at K = 600 000 it even accepts an all-zero dst); the bound the checks
apply does, as shown here with the oracle's weight.
"""
from __future__ import annotations

import numpy as np
import pytest

import out_prod_cases as cases
from gpu_util import out_prod_reference_parts
from sum_bounds import (U32, gamma, gamma_deterministic, gamma_probabilistic,
                        within_sum_bound)


def _reference(case, weight):
    n_rows, n_cols = case["n_rows"], case["n_cols"]
    b = cases.random_src1(case)
    windows = cases.row_windows(n_rows, n_cols)
    block_parts, mag = out_prod_reference_parts(weight, n_cols, b, windows)
    split = cases.smallest_split_rows(n_rows)
    last = (-(-n_rows // split) - 1) * split
    splits = [(0, split), ((n_rows // split // 2) * split, split), (last, n_rows - last)]
    split_parts, _ = out_prod_reference_parts(weight, n_cols, b, splits)
    exact = sum(block_parts, np.zeros_like(mag))
    return dict(K=n_rows, exact=exact, mag=mag, windows=windows, block_parts=block_parts,
                splits=splits, split_parts=split_parts)


@pytest.fixture(scope="module")
def pr_example():
    return _reference(cases.PR_EXAMPLE, cases.pr_example_weight())


@pytest.fixture(scope="module")
def output_head():
    return _reference(cases.OUTPUT_HEAD, cases.output_head_weight())


def _cases(request):
    return request.getfixturevalue(request.param)


@pytest.fixture(params=["pr_example", "output_head"])
def ref(request):
    return _cases(request)


def test_row_blocks_of_the_cases():
    """3 blocks for the PR's example, 13 for the output head (12 483 rows,
    the last 2 140), as the PR and the output-head workload state."""
    assert [w[1] for w in cases.row_windows(600_000, 256)] == [262_144, 262_144, 75_712]
    head = cases.row_windows(151_936, 5_376)
    assert len(head) == 13 and head[0][1] == 12_483 and head[-1][1] == 2_140


def test_the_rounded_exact_sum_passes(ref):
    got = ref["exact"].astype(np.float32)
    assert within_sum_bound(got, ref["exact"], ref["mag"], ref["K"])


def test_a_dropped_row_block_fails(ref):
    for (r0, rows), part in zip(ref["windows"], ref["block_parts"]):
        got = (ref["exact"] - part).astype(np.float32)
        assert not within_sum_bound(got, ref["exact"], ref["mag"], ref["K"]), \
            f"dropping rows [{r0}, {r0 + rows}) still passes"


def test_a_row_block_counted_twice_fails(ref):
    """A stale block added again (beta = 1 over the wrong buffer)."""
    for (r0, rows), part in zip(ref["windows"], ref["block_parts"]):
        got = (ref["exact"] + part).astype(np.float32)
        assert not within_sum_bound(got, ref["exact"], ref["mag"], ref["K"]), \
            f"counting rows [{r0}, {r0 + rows}) twice still passes"


def test_a_dropped_fused_split_fails(ref):
    """The fused route's smallest split (64 splits): the first, a middle and
    the last one."""
    for (r0, rows), part in zip(ref["splits"], ref["split_parts"]):
        got = (ref["exact"] - part).astype(np.float32)
        assert not within_sum_bound(got, ref["exact"], ref["mag"], ref["K"]), \
            f"dropping split rows [{r0}, {r0 + rows}) still passes"


def test_zero_fails_but_passes_the_deterministic_bound_at_the_pr_size(pr_example):
    """Why the checks do not use gamma_K alone: at K = 600 000 it accepts 0."""
    zero = np.zeros_like(pr_example["exact"], dtype=np.float32)
    K = pr_example["K"]
    assert not within_sum_bound(zero, pr_example["exact"], pr_example["mag"], K)
    det = gamma_deterministic(K) * pr_example["mag"]
    assert (np.abs(pr_example["exact"]) <= det).all()


def test_gamma_closed_forms():
    """gamma_K = K u / (1 - K u); the probabilistic bound ~ lam sqrt(K) u
    for K u << 1, and the smaller of the two is applied."""
    assert gamma_deterministic(1) == pytest.approx(U32 / (1 - U32), rel=1e-15)
    assert gamma_deterministic(600_000) == pytest.approx(600_000 / (2 ** 24 - 600_000),
                                                          rel=1e-14)
    assert gamma_probabilistic(10 ** 6, 8.0) == pytest.approx(8e3 * U32, rel=1e-3)
    assert gamma(4) == gamma_deterministic(4)          # small K: the deterministic one
    assert gamma(600_000) == gamma_probabilistic(600_000)


@pytest.mark.parametrize("K", [1_000, 100_000, 600_000])
@pytest.mark.parametrize("signs", ["random", "positive"])
def test_recursive_fp32_sums_stay_within_the_bound(K, signs):
    """The bound checked on the CPU against an FP32 summation whose error
    is known to grow fastest, the sequential one (numpy's cumulative sum adds
    in order): over 16 trials of K products a * w (a standard normal, or its
    absolute value; w uniform in [0, 0.05)), the error stays within
    gamma(K) * sum |a w|.  With same-sign terms the error reaches a few
    percent of the bound or more (measured 0.05-0.27 of it), so the bound is
    not loose by orders of magnitude where errors add up."""
    rng = np.random.Generator(np.random.PCG64(K))
    ratios = []
    for _ in range(16):
        a = rng.standard_normal(K).astype(np.float32)
        if signs == "positive":
            a = np.abs(a)
        w = (rng.random(K) * 0.05).astype(np.float32)
        prod = a * w                                   # FP32 products, rounded once each
        computed = np.cumsum(prod, dtype=np.float32)[-1]
        exact = np.sum(prod.astype(np.float64))
        mag = np.sum(np.abs(prod.astype(np.float64)))
        ratios.append(abs(float(computed) - exact) / (gamma(K) * mag))
    assert max(ratios) <= 1.0
    if signs == "positive":
        assert max(ratios) > 0.02
