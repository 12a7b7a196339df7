"""MI355X (gfx950) nested block-wise 4-bit dequantization.

Thin Python binding of the C ABI in include/dq4.h (libdq4.so, built in-tree
by block_wise_bit_amd/build.py).  The functions keep the C names; they only
check and marshal arguments -- every step of the dequantization runs in the
HIP kernels of the library.  torch provides device memory and the current
stream, nothing else.  There is no fallback: if the library is missing or
cannot be loaded, every call raises.

    dq4_nested_dequant(packed, scale_codes, nested_absmax, scale_codebook,
                       codebook4, offset, n, blocksize, ...) -> tensor
    dq4_nested_dequant_rows(..., n_rows, n_cols, r0, rows, ...) -> tensor
    nested_dequant(..., n, blocksize=64, dtype=None, out=None, rows=None) -> tensor
                                                   (either of the two above, torch-style)
    dq4_rows_per_block(n_cols, elem_bytes, budget_bytes) -> int
    dq4_row_window(n_rows, n_cols, elem_bytes, budget_bytes, k) -> (count, r0, rows)
    dq4_row_windows(n_rows, n_cols, elem_bytes, budget_bytes) -> [(r0, rows)]
    dq4_nested_dequant_unfused(...) -> tensor     (three-launch comparison baseline)
    dq4_nested_dequant_unfused_noalloc(...) -> tensor  (the same, scratch inside the library)
    dq4_unfused_workspace_bytes(n, blocksize) -> int
    dq4_out_prod_rows(..., n_rows, n_cols, blocksize, src1, ...) -> tensor
                                                   (row-blocked out_prod, FP32 GEMM)
    dq4_out_prod_fused(..., n_rows, n_cols, blocksize, src1, ...) -> tensor
                                                   (out_prod, dequantization in the GEMM)
    dq4_out_prod_fused_workspace_bytes(n_rows, n_cols, m, src1_transposed=False) -> int
    dq4_dequant_linear(..., n_out, n_in, blocksize, x, op) -> tensor
                                                   (Y = X W^T or G W, FP16/BF16 GEMM)
    dq4_int8_prep(A, CB, SCB, cols) -> (subA, subB)  (LLM.int8 correction operands)
    dq4_memory_twin_f16(packed, n) -> tensor       (diagnostic: the FP16 call's memory
                                                   traffic without its arithmetic)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import List, Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(PKG_DIR, "libdq4.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "dq4.h")

DQ4_OK, DQ4_EINVAL, DQ4_EUNSUPPORTED, DQ4_EHIP, DQ4_EBLAS, DQ4_ESCRATCH = 0, 1, 2, 3, 4, 5
DQ4_NOALLOC_MAX_BLOCKS = 1 << 23   # outer blocks the no-allocation call's static scratch holds
DQ4_F32, DQ4_F16, DQ4_BF16 = 0, 1, 2
DQ4_LINEAR_FORWARD, DQ4_LINEAR_GRAD_A = 0, 1
NESTED_BLOCKSIZE = 256
ROW_BLOCK_BUDGET_BYTES = 256 << 20   # 256 MiB of F32 per transient row block

_lib = None


class Dq4Error(RuntimeError):
    """A launch failure reported by the library (DQ4_EHIP)."""


def library() -> ctypes.CDLL:
    """The loaded libdq4.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY_PATH):
        raise RuntimeError(
            f"{LIBRARY_PATH} is missing: build it with `python -m block_wise_bit_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIBRARY_PATH)
    P = ctypes.c_void_p
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.dq4_nested_dequant.argtypes = [P, P, P, P, P, f32, i64, i32, i32, i32, P, P]
    lib.dq4_nested_dequant.restype = i32
    lib.dq4_nested_dequant_rows.argtypes = [P, P, P, P, P, f32, i64, i64, i64, i64, i32, i32,
                                            i32, P, P]
    lib.dq4_nested_dequant_rows.restype = i32
    lib.dq4_memory_twin_f16.argtypes = [P, i64, P, P]
    lib.dq4_memory_twin_f16.restype = i32
    lib.dq4_rows_per_block.argtypes = [i64, i64, i64]
    lib.dq4_rows_per_block.restype = i64
    lib.dq4_row_window.argtypes = [i64, i64, i64, i64, i64, P, P]
    lib.dq4_row_window.restype = i64
    lib.dq4_nested_dequant_unfused.argtypes = [P, P, P, P, P, f32, i64, i32, i32, i32, P, P, P]
    lib.dq4_nested_dequant_unfused.restype = i32
    lib.dq4_nested_dequant_unfused_noalloc.argtypes = [P, P, P, P, P, f32, i64, i32, i32, i32,
                                                       P, P]
    lib.dq4_nested_dequant_unfused_noalloc.restype = i32
    lib.dq4_unfused_workspace_bytes.argtypes = [i64, i32]
    lib.dq4_unfused_workspace_bytes.restype = i64
    lib.dq4_out_prod_rows.argtypes = [P, P, P, P, P, f32, i64, i64, i32, i32, P, i64, i64, i32, P,
                                      P, i64, P]
    lib.dq4_out_prod_rows.restype = i32
    lib.dq4_out_prod_fused.argtypes = lib.dq4_out_prod_rows.argtypes
    lib.dq4_out_prod_fused.restype = i32
    lib.dq4_out_prod_fused_workspace_bytes.argtypes = [i64, i64, i64, i32]
    lib.dq4_out_prod_fused_workspace_bytes.restype = i64
    lib.dq4_dequant_linear.argtypes = [P, P, P, P, P, f32, i64, i64, i32, i32, i32, i32, P, i64,
                                       P, P, P]
    lib.dq4_dequant_linear.restype = i32
    lib.dq4_int8_prep.argtypes = [P, i64, i64, P, P, i64, P, i64, P, P, P]
    lib.dq4_int8_prep.restype = i32
    lib.dq4_last_blas_status.argtypes = []
    lib.dq4_last_blas_status.restype = i32
    lib.dq4_status_string.argtypes = [i32]
    lib.dq4_status_string.restype = ctypes.c_char_p
    lib.dq4_last_hip_error.argtypes = []
    lib.dq4_last_hip_error.restype = i32
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> List[str]:
    """Names of the functions include/dq4.h declares."""
    with open(path) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(dq4_[a-z0-9_]+)\s*\(", text)


# ----------------------------------------------------------------------------
# plain C entry points
# ----------------------------------------------------------------------------
def dq4_status_string(status: int) -> str:
    return library().dq4_status_string(int(status)).decode()


def dq4_last_hip_error() -> int:
    return int(library().dq4_last_hip_error())


def dq4_last_blas_status() -> int:
    return int(library().dq4_last_blas_status())


def dq4_rows_per_block(n_cols: int, elem_bytes: int = 4,
                       budget_bytes: int = ROW_BLOCK_BUDGET_BYTES) -> int:
    return int(library().dq4_rows_per_block(int(n_cols), int(elem_bytes), int(budget_bytes)))


def dq4_unfused_workspace_bytes(n: int, blocksize: int) -> int:
    return int(library().dq4_unfused_workspace_bytes(int(n), int(blocksize)))


def dq4_row_window(n_rows: int, n_cols: int, elem_bytes: int, budget_bytes: int,
                   k: int) -> Tuple[int, int, int]:
    """(window count, r0, rows) of window k, from the C call of the same name;
    r0 and rows are -1 when k is not a window index."""
    r0, rows = ctypes.c_int64(-1), ctypes.c_int64(-1)
    count = library().dq4_row_window(int(n_rows), int(n_cols), int(elem_bytes),
                                     int(budget_bytes), int(k), ctypes.byref(r0),
                                     ctypes.byref(rows))
    return int(count), int(r0.value), int(rows.value)


def dq4_row_windows(n_rows: int, n_cols: int, elem_bytes: int = 4,
                    budget_bytes: int = ROW_BLOCK_BUDGET_BYTES) -> List[Tuple[int, int]]:
    """The whole row-window plan [(r0, rows), ...], window by window from
    dq4_row_window."""
    count = dq4_row_window(n_rows, n_cols, elem_bytes, budget_bytes, -1)[0]
    return [dq4_row_window(n_rows, n_cols, elem_bytes, budget_bytes, k)[1:]
            for k in range(count)]


def _raise_for(status: int, what: str) -> None:
    if status == DQ4_OK:
        return
    msg = f"{what}: {dq4_status_string(status)}"
    if status == DQ4_EHIP:
        raise Dq4Error(f"{msg} (hip error {dq4_last_hip_error()})")
    if status == DQ4_EBLAS:
        raise Dq4Error(f"{msg} (rocblas status {dq4_last_blas_status()})")
    raise ValueError(msg)


# ----------------------------------------------------------------------------
# torch-tensor forms (allocating, or writing into `out`)
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _out_code(dtype) -> int:
    torch = _torch()
    codes = {torch.float32: DQ4_F32, torch.float16: DQ4_F16, torch.bfloat16: DQ4_BF16}
    if dtype not in codes:
        raise ValueError(f"unsupported output dtype {dtype}")
    return codes[dtype]


def _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                  end: int, blocksize: int, nested_blocksize: int):
    torch = _torch()
    tensors = (packed, scale_codes, nested_absmax, scale_codebook, codebook4)
    device = packed.device
    if device.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    for name, t, dt in zip(("packed", "scale_codes", "nested_absmax", "scale_codebook",
                            "codebook4"), tensors,
                           (torch.uint8, torch.uint8, torch.float32, torch.float32,
                            torch.float32)):
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if scale_codebook.numel() != 256:
        raise ValueError("scale_codebook must hold 256 values")
    if codebook4.numel() != 16:
        raise ValueError("codebook4 must hold 16 values")
    if end > 0 and blocksize > 0 and nested_blocksize > 0:
        nb = -(-end // blocksize)
        ng = -(-nb // nested_blocksize)
        if packed.numel() < -(-end // 2):
            raise ValueError(f"packed holds {packed.numel()} bytes, needs {-(-end // 2)}")
        if scale_codes.numel() < nb:
            raise ValueError(f"scale_codes holds {scale_codes.numel()} codes, needs {nb}")
        if nested_absmax.numel() < ng:
            raise ValueError(f"nested_absmax holds {nested_absmax.numel()} values, needs {ng}")
    return device


def _prepare_out(out, count: int, dtype, device, stream=None):
    torch = _torch()
    if out is None:
        return _used_on(torch.empty(count, dtype=dtype, device=device), stream)
    if out.device != device or out.dtype != dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of the output dtype on the inputs' device")
    if out.numel() < count:
        raise ValueError(f"out holds {out.numel()} elements, needs {count}")
    return out


def _used_on(t, stream):
    """Tell torch's caching allocator that the kernels enqueued on `stream`
    use t, a tensor this module allocated on the current stream: when t is
    freed, its memory is not handed to a new allocation until that stream's
    work queued so far has finished.  Without it a temporary freed on return
    could be reused by work on the current stream while a kernel on another
    stream still reads or writes it.  (Nothing to do for the current stream,
    whose order already covers it.)"""
    if stream is not None and t.numel() > 0:
        t.record_stream(stream)
    return t


def _stream_handle(device, stream) -> ctypes.c_void_p:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def dq4_nested_dequant(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                       offset: float, n: int, blocksize: int,
                       nested_blocksize: int = NESTED_BLOCKSIZE, out_dtype=None,
                       out=None, stream=None):
    """Dequantize the first n elements; returns `out` (allocated when None).

    Enqueued on `stream` (default: torch's current stream on the inputs'
    device); asynchronous like any kernel launch.
    """
    torch = _torch()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    code = _out_code(out_dtype)
    device = _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                           int(n), int(blocksize), int(nested_blocksize))
    out = _prepare_out(out, max(int(n), 0), out_dtype, device, stream)
    with torch.cuda.device(device):
        st = library().dq4_nested_dequant(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), int(n),
            int(blocksize), int(nested_blocksize), code, out.data_ptr(),
            _stream_handle(device, stream))
    _raise_for(st, "dq4_nested_dequant")
    return out


def dq4_nested_dequant_rows(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                            offset: float, n_rows: int, n_cols: int, r0: int, rows: int,
                            blocksize: int, nested_blocksize: int = NESTED_BLOCKSIZE,
                            out_dtype=None, out=None, stream=None):
    """Dequantize rows [r0, r0+rows) of an n_rows x n_cols weight into rows*n_cols elements."""
    torch = _torch()
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    code = _out_code(out_dtype)
    n_rows, n_cols, r0, rows = int(n_rows), int(n_cols), int(r0), int(rows)
    if n_rows < 0 or n_cols < 0 or r0 < 0 or rows < 0 or r0 + rows > n_rows:
        raise ValueError(f"row window [{r0}, {r0 + rows}) outside 0..{n_rows}")
    device = _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                           (r0 + rows) * n_cols, int(blocksize), int(nested_blocksize))
    out = _prepare_out(out, rows * n_cols, out_dtype, device, stream)
    with torch.cuda.device(device):
        st = library().dq4_nested_dequant_rows(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), n_rows,
            n_cols, r0, rows, int(blocksize), int(nested_blocksize), code, out.data_ptr(),
            _stream_handle(device, stream))
    _raise_for(st, "dq4_nested_dequant_rows")
    return out


def nested_dequant(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                   offset: float, n: int, blocksize: int = 64, dtype=None, out=None,
                   rows=None, stream=None):
    """The torch-facing form of the two dequantization calls.

    rows=None: the whole flat tensor of n elements (dq4_nested_dequant).
    rows=(n_rows, n_cols, r0, count): rows [r0, r0 + count) of the
    n_rows x n_cols weight, n == n_rows * n_cols (dq4_nested_dequant_rows).
    dtype defaults to torch.float16.  out=None allocates the result; a given
    out is written in place and returned.  Bad arguments and unsupported
    layouts raise ValueError, a failed launch Dq4Error (a RuntimeError).
    """
    torch = _torch()
    dtype = torch.float16 if dtype is None else dtype
    if rows is None:
        return dq4_nested_dequant(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                                  offset, n, blocksize, out_dtype=dtype, out=out, stream=stream)
    n_rows, n_cols, r0, count = (int(v) for v in rows)
    if n_rows * n_cols != int(n):
        raise ValueError(f"rows={tuple(rows)} describes {n_rows}x{n_cols} elements, not n={n}")
    return dq4_nested_dequant_rows(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                                   offset, n_rows, n_cols, r0, count, blocksize,
                                   out_dtype=dtype, out=out, stream=stream)


def dq4_nested_dequant_unfused(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                               offset: float, n: int, blocksize: int,
                               nested_blocksize: int = NESTED_BLOCKSIZE, out_dtype=None,
                               out=None, scale_workspace=None, stream=None):
    """The unfused three-launch sequence (comparison baseline); same results as
    dq4_nested_dequant.  `scale_workspace` (FP32, >= ceil(n/blocksize)
    values) is allocated when None."""
    torch = _torch()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    code = _out_code(out_dtype)
    device = _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                           int(n), int(blocksize), int(nested_blocksize))
    out = _prepare_out(out, max(int(n), 0), out_dtype, device, stream)
    need = dq4_unfused_workspace_bytes(int(n), int(blocksize)) // 4
    if scale_workspace is None:
        scale_workspace = _used_on(torch.empty(max(need, 1), dtype=torch.float32,
                                               device=device), stream)
    elif (scale_workspace.device != device or scale_workspace.dtype != torch.float32
          or not scale_workspace.is_contiguous() or scale_workspace.numel() < need):
        raise ValueError(f"scale_workspace must be a contiguous float32 tensor of >= {need} "
                         "values on the inputs' device")
    with torch.cuda.device(device):
        st = library().dq4_nested_dequant_unfused(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), int(n),
            int(blocksize), int(nested_blocksize), code, scale_workspace.data_ptr(),
            out.data_ptr(), _stream_handle(device, stream))
    _raise_for(st, "dq4_nested_dequant_unfused")
    return out


def dq4_nested_dequant_unfused_noalloc(packed, scale_codes, nested_absmax, scale_codebook,
                                       codebook4, offset: float, n: int, blocksize: int,
                                       nested_blocksize: int = NESTED_BLOCKSIZE, out_dtype=None,
                                       out=None, stream=None):
    """The unfused sequence with its FP32 scales in the library's static
    scratch instead of a workspace: the C call allocates nothing.  Pass `out`
    to allocate nothing here either (e.g. under graph capture).  At most
    DQ4_NOALLOC_MAX_BLOCKS outer blocks; calls that overlap on one GPU race."""
    torch = _torch()
    out_dtype = torch.float16 if out_dtype is None else out_dtype
    code = _out_code(out_dtype)
    device = _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                           int(n), int(blocksize), int(nested_blocksize))
    out = _prepare_out(out, max(int(n), 0), out_dtype, device, stream)
    with torch.cuda.device(device):
        st = library().dq4_nested_dequant_unfused_noalloc(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), int(n),
            int(blocksize), int(nested_blocksize), code, out.data_ptr(),
            _stream_handle(device, stream))
    _raise_for(st, "dq4_nested_dequant_unfused_noalloc")
    return out


def _out_prod_operands(torch, packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                       n_rows, n_cols, blocksize, nested_blocksize, src1, src1_transposed, dst,
                       stream):
    """Checked (device, m, ld, dst) for the two out_prod entry points."""
    device = _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                           n_rows * n_cols, int(blocksize), int(nested_blocksize))
    if src1.device != device or src1.dtype != torch.float32 or src1.dim() != 2:
        raise ValueError("src1 must be a 2-D float32 tensor on the inputs' device")
    if src1.stride(1) != 1 and src1.size(1) > 1:
        raise ValueError("src1 must have unit stride along its last dimension")
    m = int(src1.size(0) if src1_transposed else src1.size(1))
    k_dim = int(src1.size(1) if src1_transposed else src1.size(0))
    if k_dim != n_rows:
        raise ValueError(f"src1 has {k_dim} rows of the summed dimension, the weight {n_rows}")
    # a single row's stride is arbitrary (numpy and torch leave it so): its
    # leading dimension is then the row length
    ld = max(int(src1.stride(0)) if src1.size(0) > 1 else int(src1.size(1)), 1)
    if dst is None:
        dst = _used_on(torch.empty((m, n_cols), dtype=torch.float32, device=device), stream)
    elif (dst.device != device or dst.dtype != torch.float32 or not dst.is_contiguous()
          or dst.numel() < m * n_cols):
        raise ValueError("dst must be a contiguous float32 tensor of m * n_cols values")
    return device, m, ld, dst


def _f32_workspace(torch, workspace, device):
    if (workspace.device != device or workspace.dtype != torch.float32
            or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous float32 tensor on the inputs' device")
    return workspace


def dq4_out_prod_rows(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                      offset: float, n_rows: int, n_cols: int, blocksize: int, src1,
                      src1_transposed: bool = False, dst=None, workspace=None,
                      workspace_bytes: int = ROW_BLOCK_BUDGET_BYTES,
                      nested_blocksize: int = NESTED_BLOCKSIZE, stream=None):
    """dst[i][j] = sum_r B[r][i] * W[r][j] for the nested 4-bit weight W
    (n_rows x n_cols), dequantized to FP32 in row windows of at most
    `workspace_bytes` and accumulated by an FP32 GEMM per window.

    src1 is FP32, 2-D with unit stride along its last dimension: shape
    (n_rows, m) (B = src1) or, with src1_transposed, (m, n_rows) (B = src1^T).
    Returns dst (m x n_cols, FP32).  `workspace` (FP32, at least one row of
    n_cols) is allocated when None, sized min(workspace_bytes, whole weight).
    """
    torch = _torch()
    n_rows, n_cols = int(n_rows), int(n_cols)
    device, m, ld, dst = _out_prod_operands(
        torch, packed, scale_codes, nested_absmax, scale_codebook, codebook4, n_rows, n_cols,
        blocksize, nested_blocksize, src1, src1_transposed, dst, stream)
    if workspace is None:
        rows = max(1, min(n_rows, int(workspace_bytes) // max(4 * n_cols, 1)))
        workspace = _used_on(torch.empty(max(rows * n_cols, 1), dtype=torch.float32,
                                         device=device), stream)
    workspace = _f32_workspace(torch, workspace, device)
    with torch.cuda.device(device):
        st = library().dq4_out_prod_rows(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), n_rows,
            n_cols, int(blocksize), int(nested_blocksize), src1.data_ptr(), m, ld,
            1 if src1_transposed else 0, dst.data_ptr(), workspace.data_ptr(),
            workspace.numel() * 4, _stream_handle(device, stream))
    _raise_for(st, "dq4_out_prod_rows")
    return dst


def dq4_out_prod_fused_workspace_bytes(n_rows: int, n_cols: int, m: int, device=None,
                                       src1_transposed: bool = False) -> int:
    """Workspace bytes for dq4_out_prod_fused's preferred row split on
    `device` (default: the current device) with a src1 of this orientation
    (for a transposed one, with its row-major copy); 0 when it prefers one
    split."""
    torch = _torch()
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        return int(library().dq4_out_prod_fused_workspace_bytes(
            int(n_rows), int(n_cols), int(m), 1 if src1_transposed else 0))


def dq4_out_prod_fused(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                       offset: float, n_rows: int, n_cols: int, blocksize: int, src1,
                       src1_transposed: bool = False, dst=None, workspace=None,
                       nested_blocksize: int = NESTED_BLOCKSIZE, stream=None):
    """The same sum as dq4_out_prod_rows, with the 4-bit weight decoded inside
    an FP32 matrix-core GEMM (no dequantized copy in HBM).  `workspace`
    (FP32, for partial sums over row splits and, for a transposed src1, its
    row-major copy) is allocated at the preferred size for src1's
    orientation when None; an empty tensor means one split and a transposed
    src1 read in place.  Returns dst."""
    torch = _torch()
    n_rows, n_cols = int(n_rows), int(n_cols)
    device, m, ld, dst = _out_prod_operands(
        torch, packed, scale_codes, nested_absmax, scale_codebook, codebook4, n_rows, n_cols,
        blocksize, nested_blocksize, src1, src1_transposed, dst, stream)
    if workspace is None:
        nbytes = dq4_out_prod_fused_workspace_bytes(n_rows, n_cols, m, device,
                                                    src1_transposed=src1_transposed)
        workspace = _used_on(torch.empty(max(nbytes // 4, 0), dtype=torch.float32,
                                         device=device), stream)
    workspace = _f32_workspace(torch, workspace, device)
    with torch.cuda.device(device):
        st = library().dq4_out_prod_fused(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), n_rows,
            n_cols, int(blocksize), int(nested_blocksize), src1.data_ptr(), m, ld,
            1 if src1_transposed else 0, dst.data_ptr(),
            workspace.data_ptr() if workspace.numel() else None, workspace.numel() * 4,
            _stream_handle(device, stream))
    _raise_for(st, "dq4_out_prod_fused")
    return dst


def dq4_dequant_linear(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                       offset: float, n_out: int, n_in: int, blocksize: int, x,
                       op: str = "forward", y=None, w_workspace=None,
                       nested_blocksize: int = NESTED_BLOCKSIZE, stream=None):
    """Dequantize the n_out x n_in weight W whole (into w_workspace, allocated
    when None) and run one GEMM: op "forward" gives Y = X W^T (x: m x n_in),
    op "grad_a" gives Y = G W (x: m x n_out).  x's dtype (float16 or
    bfloat16) is the dtype of W and Y.  Returns Y."""
    torch = _torch()
    n_out, n_in = int(n_out), int(n_in)
    ops = {"forward": DQ4_LINEAR_FORWARD, "grad_a": DQ4_LINEAR_GRAD_A}
    if op not in ops:
        raise ValueError("op must be 'forward' or 'grad_a'")
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("x must be float16 or bfloat16")
    code = _out_code(x.dtype)
    device = _check_inputs(packed, scale_codes, nested_absmax, scale_codebook, codebook4,
                           n_out * n_in, int(blocksize), int(nested_blocksize))
    k = n_in if op == "forward" else n_out
    width = n_out if op == "forward" else n_in
    if x.device != device or x.dim() != 2 or x.size(1) != k or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous (m, {k}) tensor on the inputs' device")
    m = int(x.size(0))
    if y is None:
        y = _used_on(torch.empty((m, width), dtype=x.dtype, device=device), stream)
    elif y.device != device or y.dtype != x.dtype or not y.is_contiguous() or y.numel() < m * width:
        raise ValueError(f"y must be a contiguous {x.dtype} tensor of {m} x {width} values")
    if w_workspace is None:
        w_workspace = _used_on(torch.empty(max(n_out * n_in, 1), dtype=x.dtype, device=device),
                               stream)
    elif (w_workspace.device != device or w_workspace.dtype != x.dtype
          or not w_workspace.is_contiguous() or w_workspace.numel() < n_out * n_in):
        raise ValueError("w_workspace must hold n_out * n_in values of x's dtype")
    with torch.cuda.device(device):
        st = library().dq4_dequant_linear(
            packed.data_ptr(), scale_codes.data_ptr(), nested_absmax.data_ptr(),
            scale_codebook.data_ptr(), codebook4.data_ptr(), ctypes.c_float(offset), n_out,
            n_in, int(blocksize), int(nested_blocksize), code, ops[op], x.data_ptr(), m,
            y.data_ptr(), w_workspace.data_ptr(), _stream_handle(device, stream))
    _raise_for(st, "dq4_dequant_linear")
    return y


def dq4_int8_prep(A, CB, SCB, cols, subA=None, subB=None, stream=None, validate=False):
    """LLM.int8 correction operands in one kernel: subA = A[:, cols] (M x L,
    FP16) and subB = fp16(fl32(fl32(CB[:, cols] * SCB[:, None]) * R127)).T
    (L x N, FP16, contiguous).

    Asynchronous and capturable into a HIP graph: the kernel itself never
    reads through a column index outside [0, K) and sets the outputs such an
    index feeds to FP16 NaN.  validate=True also checks the indices on the
    host first, raising ValueError for an out-of-range one; that check reads
    them back, a synchronization on every call, so it is off by default."""
    torch = _torch()
    device = A.device
    if device.type != "cuda":
        raise ValueError("A must be a GPU tensor")
    if A.dtype != torch.float16 or A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be a contiguous 2-D float16 tensor")
    if CB.dtype != torch.int8 or CB.dim() != 2 or not CB.is_contiguous():
        raise ValueError("CB must be a contiguous 2-D int8 tensor")
    if SCB.dtype != torch.float32 or SCB.dim() != 1 or not SCB.is_contiguous():
        raise ValueError("SCB must be a contiguous 1-D float32 tensor")
    if cols.dtype != torch.int64 or cols.dim() != 1 or not cols.is_contiguous():
        raise ValueError("cols must be a contiguous 1-D int64 tensor")
    for name, t in (("CB", CB), ("SCB", SCB), ("cols", cols)):
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
    M, K = A.shape
    N = CB.shape[0]
    if CB.shape[1] != K or SCB.numel() != N:
        raise ValueError(f"CB must be N x {K} and SCB must hold N values")
    L = cols.numel()
    if validate and L and bool(((cols < 0) | (cols >= K)).any()):
        raise ValueError(f"column indices must lie in [0, {K})")
    if subA is None:
        subA = _used_on(torch.empty((M, L), dtype=torch.float16, device=device), stream)
    if subB is None:
        subB = _used_on(torch.empty((L, N), dtype=torch.float16, device=device), stream)
    for name, t, numel in (("subA", subA, M * L), ("subB", subB, L * N)):
        if (t.device != device or t.dtype != torch.float16 or not t.is_contiguous()
                or t.numel() < numel):
            raise ValueError(f"{name} must be a contiguous float16 tensor of {numel} values")
    with torch.cuda.device(device):
        st = library().dq4_int8_prep(A.data_ptr(), M, K, CB.data_ptr(), SCB.data_ptr(), N,
                                     cols.data_ptr(), L, subA.data_ptr(), subB.data_ptr(),
                                     _stream_handle(device, stream))
    _raise_for(st, "dq4_int8_prep")
    return subA, subB


def dq4_memory_twin_f16(packed, n: int, out=None, stream=None):
    """Diagnostic: the FP16 call's memory traffic without its arithmetic (see
    include/dq4.h).  `out` (or the returned tensor) holds 2n bytes as n
    float16 slots; as uint32, out[4u + i] = packed word u."""
    torch = _torch()
    if packed.device.type != "cuda" or packed.dtype != torch.uint8 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous uint8 GPU tensor")
    if packed.numel() < -(-int(n) // 2):
        raise ValueError(f"packed holds {packed.numel()} bytes, needs {-(-int(n) // 2)}")
    out = _prepare_out(out, max(int(n), 0), torch.float16, packed.device, stream)
    with torch.cuda.device(packed.device):
        st = library().dq4_memory_twin_f16(packed.data_ptr(), int(n), out.data_ptr(),
                                           _stream_handle(packed.device, stream))
    _raise_for(st, "dq4_memory_twin_f16")
    return out


def to_device(x, device="cuda"):
    """Upload host inputs (block_wise_bit_amd.inputs.NestedInputs) as GPU tensors."""
    torch = _torch()
    return dict(
        packed=torch.from_numpy(x.packed).to(device),
        scale_codes=torch.from_numpy(x.scale_codes).to(device),
        nested_absmax=torch.from_numpy(x.nested_absmax).to(device),
        scale_codebook=torch.from_numpy(x.scale_codebook).to(device),
        codebook4=torch.from_numpy(x.codebook4).to(device),
    )
