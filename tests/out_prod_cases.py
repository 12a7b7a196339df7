"""Inputs of the full-size out_prod checks, shared by the GPU tests and the
CPU negative controls that show those checks can fail (no arithmetic of the
method lives here).

llama.cpp PR "cuda: out_prod dequantizes a 2D weight in row blocks": its
worked example is 600 000 rows at 256 columns, which dequantizes in three
256 MiB F32 row blocks, and the approving review says only those multi-block
cases show a wrong k-offset or a missing beta = 1.  The output head
(151 936 x 5 376) takes 13 such blocks.
"""
from __future__ import annotations

import numpy as np

from block_wise_bit_amd import inputs

ROW_BLOCK_BUDGET = 256 << 20   # bytes of F32 per row block
MAX_FUSED_SPLITS = 64          # the fused route splits its rows at most this many ways

PR_EXAMPLE = dict(n_rows=600_000, n_cols=256, m=8, src1_seed=1)
OUTPUT_HEAD = dict(n_rows=inputs.OUTPUT_HEAD.n_rows, n_cols=inputs.OUTPUT_HEAD.n_cols, m=16,
                   src1_seed=3)


def pr_example_weight():
    n_rows, n_cols = PR_EXAMPLE["n_rows"], PR_EXAMPLE["n_cols"]
    return inputs.make_inputs(n_rows * n_cols, 64, "nf4", 0.03, seed=600_000, n_rows=n_rows,
                              n_cols=n_cols)


def output_head_weight():
    return inputs.OUTPUT_HEAD.inputs()


def random_src1(case) -> np.ndarray:
    """Standard-normal FP32 src1 of the case, stored n_rows x m."""
    rng = np.random.Generator(np.random.PCG64(case["src1_seed"]))
    return rng.standard_normal((case["n_rows"], case["m"])).astype(np.float32)


def row_windows(n_rows: int, n_cols: int, budget: int = ROW_BLOCK_BUDGET):
    """The row blocks (r0, rows) of at most budget // (4 n_cols) rows."""
    rpb = max(1, budget // (4 * n_cols))
    return [(r0, min(rpb, n_rows - r0)) for r0 in range(0, n_rows, rpb)]


def smallest_split_rows(n_rows: int) -> int:
    """Rows of a fused-route split at the most splits it takes (a multiple of
    its 16-row stage)."""
    per = -(-n_rows // MAX_FUSED_SPLITS)
    return -(-per // 16) * 16


def target_rows(n_rows: int, windows, points: int = 128):
    """Weight rows a selection-matrix src1 must pick so that every row block
    and every fused-route row split holds at least one: `points` evenly spaced
    rows (spacing n_rows / points, below the smallest split when points >
    MAX_FUSED_SPLITS), the first and last row, and both rows at every block
    edge."""
    rows = {int((k + 0.5) * n_rows / points) for k in range(points)}
    rows |= {0, n_rows - 1}
    for r0, count in windows:
        rows |= {r0, r0 + count - 1}
    return sorted(r for r in rows if 0 <= r < n_rows)


def selection_groups(rows, m: int):
    """rows cut into consecutive groups of m (the last padded by repeating its
    first rows): one selection-matrix call per group."""
    groups = []
    for k in range(0, len(rows), m):
        g = list(rows[k:k + m])
        while len(g) < m:
            g.append(g[len(g) % max(1, len(rows[k:k + m]))])
        groups.append(np.array(g, dtype=np.int64))
    return groups


def selection_src1(n_rows: int, sel) -> np.ndarray:
    """B[r][i] = 1 if r == sel[i] else 0, stored n_rows x len(sel)."""
    b = np.zeros((n_rows, len(sel)), np.float32)
    b[np.asarray(sel), np.arange(len(sel))] = 1.0
    return b
