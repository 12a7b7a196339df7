"""C ABI of libdq4.so, checked without a GPU.

The library must load, export every function include/dq4.h declares, and
reject bad arguments on the host before anything is enqueued (these calls
return before any HIP runtime call, so they run on a machine without a GPU).
"""
import ctypes
import os

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from libs import ensure_hip_library

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def lib():
    return ensure_hip_library()


def test_exports_every_declared_function(lib):
    names = dq4.header_functions()
    assert set(names) == {"dq4_nested_dequant", "dq4_nested_dequant_rows", "dq4_rows_per_block",
                          "dq4_status_string", "dq4_last_hip_error",
                          "dq4_nested_dequant_unfused", "dq4_unfused_workspace_bytes",
                          "dq4_out_prod_rows", "dq4_last_blas_status", "dq4_dequant_linear",
                          "dq4_int8_prep", "dq4_out_prod_fused",
                          "dq4_out_prod_fused_workspace_bytes", "dq4_memory_twin_f16",
                          "dq4_row_window", "dq4_nested_dequant_unfused_noalloc"}
    for name in names:
        assert hasattr(lib, name), name
    # and the binding keeps the C names
    for name in names:
        assert callable(getattr(dq4, name)), name


def test_status_strings(lib):
    for st in (dq4.DQ4_OK, dq4.DQ4_EINVAL, dq4.DQ4_EUNSUPPORTED, dq4.DQ4_EHIP, dq4.DQ4_EBLAS,
               dq4.DQ4_ESCRATCH, 99):
        s = dq4.dq4_status_string(st)
        assert s.startswith("DQ4")
    assert dq4.dq4_last_hip_error() == 0
    assert dq4.dq4_last_blas_status() == 0


def _call(lib, n=64, blocksize=64, nested=256, dtype=dq4.DQ4_F16, ptr=1, out=1):
    # fake non-null device pointers: every call here must fail validation or be a no-op
    p = ctypes.c_void_p(ptr) if ptr else None
    o = ctypes.c_void_p(out) if out else None
    return lib.dq4_nested_dequant(p, p, p, p, p, ctypes.c_float(0.03), n, blocksize, nested, dtype,
                                  o, None)


def test_validation_whole_tensor(lib):
    assert _call(lib, n=0) == dq4.DQ4_OK                          # no-op
    assert _call(lib, n=0, ptr=0, out=0) == dq4.DQ4_OK            # no-op, null pointers allowed
    assert _call(lib, n=-1) == dq4.DQ4_EINVAL
    assert _call(lib, n=(1 << 62) + 1) == dq4.DQ4_EINVAL         # beyond any tensor
    assert _call(lib, n=(1 << 63) - 1) == dq4.DQ4_EINVAL
    assert _call(lib, ptr=0) == dq4.DQ4_EINVAL
    assert _call(lib, out=0) == dq4.DQ4_EINVAL
    assert _call(lib, dtype=3) == dq4.DQ4_EINVAL
    assert _call(lib, dtype=-1) == dq4.DQ4_EINVAL
    for bs in (0, 16, 48, 100, 8192, -64):
        assert _call(lib, blocksize=bs) == dq4.DQ4_EUNSUPPORTED, bs
    for nested in (0, 128, 512):
        assert _call(lib, nested=nested) == dq4.DQ4_EUNSUPPORTED


def test_validation_unfused(lib):
    p = ctypes.c_void_p(1)

    def call(n=64, blocksize=64, nested=256, dtype=dq4.DQ4_F16, ws=p):
        return lib.dq4_nested_dequant_unfused(p, p, p, p, p, ctypes.c_float(0.0), n, blocksize,
                                              nested, dtype, ws, p, None)
    assert call(n=0) == dq4.DQ4_OK
    assert call(n=-5) == dq4.DQ4_EINVAL
    assert call(n=(1 << 63) - 1) == dq4.DQ4_EINVAL
    assert call(ws=None) == dq4.DQ4_EINVAL
    assert call(blocksize=100) == dq4.DQ4_EUNSUPPORTED
    assert call(nested=64) == dq4.DQ4_EUNSUPPORTED
    assert call(dtype=9) == dq4.DQ4_EINVAL
    assert dq4.dq4_unfused_workspace_bytes(1000, 64) == 4 * 16
    assert dq4.dq4_unfused_workspace_bytes(1024, 64) == 4 * 16
    assert dq4.dq4_unfused_workspace_bytes(1025, 64) == 4 * 17
    assert dq4.dq4_unfused_workspace_bytes(0, 64) == 0
    assert dq4.dq4_unfused_workspace_bytes((1 << 63) - 1, 64) == 0   # no overflow


def test_validation_unfused_noalloc(lib):
    """The allocation-free call rejects more outer blocks than its static
    scratch holds, before touching the GPU; other checks as for the unfused
    call."""
    p = ctypes.c_void_p(1)

    def call(n=64, blocksize=64, nested=256, dtype=dq4.DQ4_F16, out=p, ptr=p):
        return lib.dq4_nested_dequant_unfused_noalloc(ptr, p, p, p, p, ctypes.c_float(0.0), n,
                                                      blocksize, nested, dtype, out, None)
    limit = dq4.DQ4_NOALLOC_MAX_BLOCKS
    assert limit == 1 << 23
    assert call(n=0) == dq4.DQ4_OK
    assert call(n=-5) == dq4.DQ4_EINVAL
    assert call(out=None) == dq4.DQ4_EINVAL
    assert call(ptr=None) == dq4.DQ4_EINVAL
    assert call(blocksize=100) == dq4.DQ4_EUNSUPPORTED
    assert call(nested=64) == dq4.DQ4_EUNSUPPORTED
    assert call(dtype=9) == dq4.DQ4_EINVAL
    assert call(n=limit * 32 + 1, blocksize=32) == dq4.DQ4_ESCRATCH      # one block too many
    assert call(n=limit * 4096 + 1, blocksize=4096) == dq4.DQ4_ESCRATCH
    assert call(n=(1 << 62), blocksize=64) == dq4.DQ4_ESCRATCH
    assert "scratch" in dq4.dq4_status_string(dq4.DQ4_ESCRATCH)


def test_validation_out_prod(lib):
    p = ctypes.c_void_p(1)

    def call(n_rows=100, n_cols=64, m=8, ld=8, trans=0, ws_bytes=64 * 4 * 10, blocksize=64,
             ws=p, src=p, dst=p):
        return lib.dq4_out_prod_rows(p, p, p, p, p, ctypes.c_float(0.0), n_rows, n_cols, blocksize,
                                     256, src, m, ld, trans, dst, ws, ws_bytes, None)
    assert call(m=0) == dq4.DQ4_OK                    # empty dst: nothing to do
    assert call(n_cols=0) == dq4.DQ4_OK
    assert call(n_rows=-1) == dq4.DQ4_EINVAL
    assert call(m=-1) == dq4.DQ4_EINVAL
    assert call(trans=2) == dq4.DQ4_EINVAL
    assert call(ld=7) == dq4.DQ4_EINVAL               # ld < m
    assert call(trans=1, ld=99) == dq4.DQ4_EINVAL     # ld < n_rows
    assert call(ws_bytes=64 * 4 - 1) == dq4.DQ4_EINVAL  # less than one F32 row
    assert call(ws=None) == dq4.DQ4_EINVAL
    assert call(src=None) == dq4.DQ4_EINVAL
    assert call(dst=None) == dq4.DQ4_EINVAL
    assert call(m=1 << 31, ld=1 << 31) == dq4.DQ4_EINVAL   # beyond the 32-bit GEMM interface
    assert call(blocksize=7) == dq4.DQ4_EUNSUPPORTED


def test_validation_out_prod_fused(lib):
    p = ctypes.c_void_p(1)

    def call(n_rows=100, n_cols=64, m=8, ld=8, trans=0, ws_bytes=0, blocksize=64, ws=None,
             src=p, dst=p, nested=256):
        return lib.dq4_out_prod_fused(p, p, p, p, p, ctypes.c_float(0.0), n_rows, n_cols,
                                      blocksize, nested, src, m, ld, trans, dst, ws, ws_bytes,
                                      None)
    assert call(m=0) == dq4.DQ4_OK                    # empty dst: nothing to do
    assert call(n_cols=0) == dq4.DQ4_OK
    assert call(n_rows=-1) == dq4.DQ4_EINVAL
    assert call(m=-1) == dq4.DQ4_EINVAL
    assert call(trans=2) == dq4.DQ4_EINVAL
    assert call(ld=7) == dq4.DQ4_EINVAL               # ld < m
    assert call(trans=1, ld=99) == dq4.DQ4_EINVAL     # ld < n_rows
    assert call(ws_bytes=-4) == dq4.DQ4_EINVAL
    assert call(ws_bytes=1024, ws=None) == dq4.DQ4_EINVAL   # a size without a buffer
    assert call(src=None) == dq4.DQ4_EINVAL
    assert call(dst=None) == dq4.DQ4_EINVAL
    assert call(blocksize=7) == dq4.DQ4_EUNSUPPORTED
    assert call(nested=128) == dq4.DQ4_EUNSUPPORTED
    # 256-row tiles at this m: 2^31 i-tiles, more than a grid can hold
    assert call(m=(1 << 31) * 256, ld=(1 << 31) * 256) == dq4.DQ4_EUNSUPPORTED
    for args in ((0, 64, 8, 0), (100, 0, 8, 0), (100, 64, 0, 1), (-1, 64, 8, 0),
                 (1 << 40, 1 << 40, 1 << 40, 0), (100, 64, 8, 2), (1 << 60, 64, 1 << 10, 1)):
        assert lib.dq4_out_prod_fused_workspace_bytes(*args) == 0


def test_validation_linear(lib):
    p = ctypes.c_void_p(1)

    def call(n_out=64, n_in=64, m=4, dtype=dq4.DQ4_F16, op=0, x=p, y=p, ws=p, blocksize=64):
        return lib.dq4_dequant_linear(p, p, p, p, p, ctypes.c_float(0.0), n_out, n_in, blocksize,
                                      256, dtype, op, x, m, y, ws, None)
    assert call(m=0) == dq4.DQ4_OK
    assert call(n_out=0, op=0) == dq4.DQ4_OK          # forward: Y is m x 0
    assert call(n_in=0, op=1) == dq4.DQ4_OK           # grad_A: Y is m x 0
    assert call(dtype=dq4.DQ4_F32) == dq4.DQ4_EINVAL
    assert call(op=2) == dq4.DQ4_EINVAL
    assert call(m=-1) == dq4.DQ4_EINVAL
    assert call(x=None) == dq4.DQ4_EINVAL
    assert call(ws=None) == dq4.DQ4_EINVAL
    assert call(n_out=1 << 31) == dq4.DQ4_EINVAL
    assert call(blocksize=16) == dq4.DQ4_EUNSUPPORTED


def test_validation_int8_prep(lib):
    p = ctypes.c_void_p(1)

    def call(M=4, K=64, N=8, L=2, A=p, CB=p, SCB=p, cols=p, subA=p, subB=p):
        return lib.dq4_int8_prep(A, M, K, CB, SCB, N, cols, L, subA, subB, None)
    assert call(L=0) == dq4.DQ4_OK                    # the empty-outlier path: nothing launched
    assert call(L=0, A=None, CB=None, cols=None) == dq4.DQ4_OK
    assert call(M=0, N=0) == dq4.DQ4_OK
    assert call(M=-1) == dq4.DQ4_EINVAL
    assert call(L=-1) == dq4.DQ4_EINVAL
    assert call(K=0) == dq4.DQ4_EINVAL
    assert call(cols=None) == dq4.DQ4_EINVAL
    assert call(subA=None) == dq4.DQ4_EINVAL
    assert call(subB=None) == dq4.DQ4_EINVAL
    assert call(M=1 << 40, K=1 << 40) == dq4.DQ4_EINVAL   # overflows 64 bits
    assert call(M=1 << 20, K=1 << 12) == dq4.DQ4_EUNSUPPORTED   # beyond 32-bit indexing


def _call_rows(lib, n_rows=10, n_cols=64, r0=0, rows=1, blocksize=64, dtype=dq4.DQ4_F32, ptr=1):
    p = ctypes.c_void_p(ptr) if ptr else None
    return lib.dq4_nested_dequant_rows(p, p, p, p, p, ctypes.c_float(0.0), n_rows, n_cols, r0,
                                       rows, blocksize, 256, dtype, p, None)


def test_validation_rows(lib):
    assert _call_rows(lib, rows=0) == dq4.DQ4_OK
    assert _call_rows(lib, r0=10, rows=0) == dq4.DQ4_OK
    assert _call_rows(lib, n_cols=0, rows=3) == dq4.DQ4_OK
    assert _call_rows(lib, r0=-1) == dq4.DQ4_EINVAL
    assert _call_rows(lib, rows=-1) == dq4.DQ4_EINVAL
    assert _call_rows(lib, r0=9, rows=2) == dq4.DQ4_EINVAL
    assert _call_rows(lib, r0=11, rows=0) == dq4.DQ4_EINVAL
    assert _call_rows(lib, n_rows=-1) == dq4.DQ4_EINVAL
    assert _call_rows(lib, n_rows=1 << 40, n_cols=1 << 40) == dq4.DQ4_EINVAL   # overflow
    assert _call_rows(lib, n_rows=1 << 31, n_cols=(1 << 31) + 1, rows=0) == dq4.DQ4_EINVAL
    assert _call_rows(lib, ptr=0) == dq4.DQ4_EINVAL
    assert _call_rows(lib, blocksize=24) == dq4.DQ4_EUNSUPPORTED
    assert _call_rows(lib, dtype=7) == dq4.DQ4_EINVAL


def test_rows_per_block_worked_examples(lib):
    with open(os.path.join(GOLDEN, "rows_per_block.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            n_cols, elem, budget, n_rows, rpb, windows, last = (
                None if v == "-" else int(v) for v in line.split())
            got = dq4.dq4_rows_per_block(n_cols, elem, budget)
            if rpb is not None:
                assert got == rpb
            w = dq4.dq4_row_windows(n_rows, n_cols, elem, budget)
            assert len(w) == windows
            assert sum(r for _, r in w) == n_rows
            if last is not None:
                assert w[-1][1] == last
    assert dq4.dq4_rows_per_block(0, 4, 1 << 28) == 1
    assert dq4.dq4_rows_per_block(256, 4, 0) == 1


def test_row_window_plan_through_the_c_abi(lib):
    """dq4_row_window called through ctypes on the worked examples: the
    window count, consecutive windows that tile [0, n_rows), each of
    rows_per_block rows but the last; out-of-range k writes nothing."""
    with open(os.path.join(GOLDEN, "rows_per_block.txt")) as fh:
        lines = [ln.split("#", 1)[0].split() for ln in fh]
    for fields in (f for f in lines if f):
        n_cols, elem, budget, n_rows, rpb, windows, last = (
            None if v == "-" else int(v) for v in fields)
        r0, rows = ctypes.c_int64(-7), ctypes.c_int64(-7)
        count = lib.dq4_row_window(n_rows, n_cols, elem, budget, -1, ctypes.byref(r0),
                                   ctypes.byref(rows))
        assert count == windows and (r0.value, rows.value) == (-7, -7)
        assert lib.dq4_row_window(n_rows, n_cols, elem, budget, count, ctypes.byref(r0),
                                  ctypes.byref(rows)) == count
        assert (r0.value, rows.value) == (-7, -7)
        step = lib.dq4_rows_per_block(n_cols, elem, budget)
        nxt = 0
        for k in range(count):
            assert lib.dq4_row_window(n_rows, n_cols, elem, budget, k, ctypes.byref(r0),
                                      ctypes.byref(rows)) == count
            assert r0.value == nxt
            assert rows.value == (step if k < count - 1 else n_rows - nxt)
            nxt += rows.value
        assert nxt == n_rows
        if last is not None:
            assert rows.value == last
        assert lib.dq4_row_window(n_rows, n_cols, elem, budget, 0, None, None) == count
    assert lib.dq4_row_window(0, 256, 4, 1 << 28, 0, None, None) == 0
    assert lib.dq4_row_window(-5, 256, 4, 1 << 28, 0, None, None) == 0
    assert dq4.dq4_row_windows(5, 3, 4, 24) == [(0, 2), (2, 2), (4, 1)]


def test_binding_rejects_host_tensors(lib):
    torch = pytest.importorskip("torch")
    u8 = torch.zeros(64, dtype=torch.uint8)
    f = torch.zeros(256, dtype=torch.float32)
    with pytest.raises(ValueError):
        dq4.dq4_nested_dequant(u8, u8, f, f, f[:16], 0.0, 64, 64)
    with pytest.raises(ValueError):
        dq4.nested_dequant(u8, u8, f, f, f[:16], 0.0, 64)
    with pytest.raises(ValueError):
        dq4.nested_dequant(u8, u8, f, f, f[:16], 0.0, 64, rows=(8, 8, 0, 4))
    with pytest.raises(ValueError):   # the window's shape does not match n
        dq4.nested_dequant(u8, u8, f, f, f[:16], 0.0, 64, rows=(8, 9, 0, 4))


def test_product_path_does_not_reach_the_oracle():
    """The package and its build never import, load or name the oracle."""
    pkg = os.path.dirname(dq4.__file__)
    for root, _, files in os.walk(pkg):
        for fname in files:
            if fname.endswith((".py", ".hip", ".h", ".cpp")):
                with open(os.path.join(root, fname)) as fh:
                    text = fh.read()
                assert "import oracle" not in text and "from oracle" not in text, fname
                assert "dq4o_" not in text and "dq4_oracle" not in text, fname


def test_validation_memory_twin(lib):
    p = ctypes.c_void_p(16)
    assert lib.dq4_memory_twin_f16(p, 0, p, None) == dq4.DQ4_OK
    assert lib.dq4_memory_twin_f16(p, -4096, p, None) == dq4.DQ4_EINVAL
    assert lib.dq4_memory_twin_f16(p, 4095, p, None) == dq4.DQ4_EINVAL     # whole tiles only
    assert lib.dq4_memory_twin_f16(None, 4096, p, None) == dq4.DQ4_EINVAL
    assert lib.dq4_memory_twin_f16(p, 4096, ctypes.c_void_p(8), None) == dq4.DQ4_EINVAL
    assert lib.dq4_memory_twin_f16(ctypes.c_void_p(2), 4096, p, None) == dq4.DQ4_EINVAL
