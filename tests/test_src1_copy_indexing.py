"""CPU restatement of the index arithmetic of the fused out_prod's src1 copy
kernel (src1_transpose_kernel in csrc/dq4_out_prod_fused.hip), which copies
the columns of a transposed src1 (m rows of n_rows floats, leading
dimension ld) into a row-major n_rows x m matrix: out[r * m + i] =
src1[i * ld + r].  One workgroup of 256 lanes moves a 64 x 64 tile (grid x:
tiles of rows r, grid y: tiles of columns i); each lane reads 16 elements
(element k = lane + 256 q is column k / 64, row k % 64 of the tile), and
writes through runs of the next power of two of the tile's column count.
The checks: every read stays inside the m x ld source (the last row only
needs n_rows floats), every write inside the copy, each output written
exactly once, with the right source element."""
import numpy as np
import pytest

T, LANES, PER = 64, 256, 16


def emulate(n_rows, m, ld, plant=None):
    src_extent = (m - 1) * ld + n_rows
    out = np.full(n_rows * m, -1, np.int64)
    for bx in range(-(-n_rows // T)):
        for by in range(-(-m // T)):
            r0, i0 = bx * T, by * T
            nr, ni = min(T, n_rows - r0), min(T, m - i0)
            k = (np.arange(LANES)[:, None] + LANES * np.arange(PER)[None, :]).ravel()
            ii, rr = k // T, k % T
            ok = (ii < ni) & (rr < nr)
            idx = (i0 + ii[ok]) * ld + r0 + rr[ok]
            if plant == "swapped_read":
                idx = (r0 + rr[ok]) * ld + i0 + ii[ok]
            assert idx.min() >= 0 and idx.max() < src_extent
            tile = np.zeros((T, T + 1), np.int64)
            tile[ii[ok], rr[ok]] = idx                 # the source element's index
            lg = (ni - 1).bit_length()
            rr, ii = k >> lg, k & ((1 << lg) - 1)
            ok = (rr < nr) & (ii < ni) if plant != "no_column_check" else rr < nr
            o = (r0 + rr[ok]) * m + i0 + ii[ok]
            assert o.min() >= 0 and o.max() < n_rows * m
            assert (out[o] == -1).all(), "an output written twice"
            out[o] = tile[ii[ok], rr[ok]]
    r, i = np.divmod(np.arange(n_rows * m), m)
    assert (out == i * ld + r).all()


@pytest.mark.parametrize("n_rows,m,ld", [
    (4099, 2, 4099), (4099, 33, 4112), (64, 64, 64), (65, 1, 70), (151, 150, 160),
    (1, 7, 1), (300, 65, 301), (128, 64, 130), (63, 128, 63), (200, 40, 211)])
def test_copy_covers_every_element_once_and_reads_in_range(n_rows, m, ld):
    emulate(n_rows, m, ld)


@pytest.mark.parametrize("plant", ["swapped_read", "no_column_check"])
def test_planted_mistakes_fail(plant):
    """The emulation rejects a read with rows and columns swapped, and a
    write that drops the check of the tile's column count."""
    with pytest.raises(AssertionError):
        emulate(100, 5, 103, plant)
