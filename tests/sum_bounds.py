"""Error bounds for FP32 sums of products, used by the out_prod checks.

An out_prod element dst[i][j] = sum_r B[r][i] W[r][j] is an inner product of
length K = n_rows, computed in FP32 in an order the test does not control (a
library GEMM, or the fused kernel's matrix-core blocks and row splits).  Two
bounds on |computed - exact|, both relative to mag = sum_r |B[r][i]| |W[r][j]|:

* deterministic: gamma_K = K u / (1 - K u), u = 2^-24 (Higham, "Accuracy and
  Stability of Numerical Algorithms", 2nd ed., section 3.1).  It holds for
  every order, with or without fused multiply-adds, but it grows like K while
  a sum of random-sign terms grows like sqrt(K): at K = 600 000 it is about
  0.036 mag, far above |exact|, so a dst that drops a whole row window still
  passes it;
* probabilistic: gamma~_K(lam) = exp(lam sqrt(K) u + K u^2 / (1 - u)) - 1
  (Higham and Mary, "A new approach to probabilistic rounding error
  analysis", SIAM J. Sci. Comput. 41(5), 2019, the inner-product theorem of
  section 4).  It holds with probability at least 1 - 2 K exp(-lam^2 (1 - u)^2
  / 2) when the rounding errors are independent, mean-zero random variables,
  the model the paper adopts; with lam = 8 that failure probability is below
  2.6e-14 K.  It grows like sqrt(K), so it rejects a dropped window.

check_sum_bound asserts the smaller of the two.  No arithmetic of the
dequantization lives here.
"""
from __future__ import annotations

import math
import sys

import numpy as np

U32 = 2.0 ** -24      # unit roundoff of binary32
PROB_LAMBDA = 8.0     # confidence parameter of the probabilistic bound


def gamma_deterministic(K: int) -> float:
    Ku = K * U32
    return Ku / (1.0 - Ku)


def gamma_probabilistic(K: int, lam: float = PROB_LAMBDA) -> float:
    return math.expm1(lam * math.sqrt(K) * U32 + K * U32 * U32 / (1.0 - U32))


def gamma(K: int) -> float:
    """The bound check_sum_bound applies: the smaller of the two."""
    return min(gamma_deterministic(K), gamma_probabilistic(K))


def sum_bound_ratio(got, exact, mag, K, factor=1.0) -> float:
    """max over elements of |got - exact| / (factor * gamma(K) * mag)."""
    err = np.abs(np.asarray(got, dtype=np.float64) - exact)
    bound = factor * gamma(K) * mag
    return float(np.max(err / np.maximum(bound, 1e-300)))


def within_sum_bound(got, exact, mag, K, factor=1.0) -> bool:
    got = np.asarray(got)
    if not np.isfinite(got).all():
        return False
    err = np.abs(got.astype(np.float64) - exact)
    return bool((err <= factor * gamma(K) * mag).all())


def check_sum_bound(got, exact, mag, K, what, factor=1.0):
    """Every element within factor * gamma(K) * mag of the exact sum."""
    worst = sum_bound_ratio(got, exact, mag, K, factor)
    print(f"{what}: worst err/bound {worst:.3e} (gamma {gamma(K):.3e} at K = {K})", flush=True)
    sys.stdout.flush()
    assert np.isfinite(np.asarray(got)).all(), what
    assert within_sum_bound(got, exact, mag, K, factor), \
        f"{what}: error above the FP32 summation bound (worst err/bound {worst:.3e})"
