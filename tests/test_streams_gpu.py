"""Calls on a stream other than torch's current one (GPU).

The torch binding allocates temporaries (workspaces) and, when none is
given, the outputs, on the current stream, while the kernels run on the
caller's `stream`.  Each such tensor is marked as used on that stream, so
that torch's caching allocator does not hand its memory to a new allocation
on the current stream while the kernels may still read or write it.

Each test holds the side stream busy (a chain of FP32 matrix products on it),
makes one call on that stream, then -- while the side stream is still busy --
allocates tensors of the same sizes on the current stream and writes into
them.  None of them may receive the memory of a temporary the call
allocated (a control first shows that the allocator does reuse a freed block
at once when nothing is marked), and after synchronizing the call's result
must equal the oracle's (bit for bit for the dequantization, exactly for the
selection-matrix out_prod).
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from block_wise_bit_amd import inputs
from gpu_util import assert_bits_equal, bits_of, oracle_bits, say, weight_rows

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from libs import ensure_hip_library
    ensure_hip_library()


@pytest.fixture()
def recorded(monkeypatch):
    """data_ptr and size of every tensor the binding marks for a stream."""
    seen = []
    orig = dq4._used_on

    def spy(t, stream):
        if stream is not None and t.numel() > 0:
            seen.append((t.data_ptr(), t.numel(), t.dtype))
        return orig(t, stream)

    monkeypatch.setattr(dq4, "_used_on", spy)
    return seen


def busy(side, ms_hint=60):
    """Queue ~tens of milliseconds of FP32 matrix products on `side`."""
    a = torch.randn(4096, 4096, device="cuda")
    b = torch.randn(4096, 4096, device="cuda") / 64.0
    c = torch.empty_like(a)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(40):
            torch.mm(a, b, out=c)
    return a, b, c   # the caller keeps them alive until it synchronizes


def scribble_and_check(seen, side):
    """While `side` is busy: same-size allocations on the current stream
    must not get a recorded temporary's memory; fill them with NaN."""
    assert seen, "the call allocated nothing"
    assert not side.query(), "the side stream finished too early to test anything"
    junk = []
    for ptr, numel, dtype in seen:
        for _ in range(2):
            t = torch.empty(numel, dtype=dtype, device="cuda")
            assert t.data_ptr() != ptr, "a temporary in use on the side stream was reused"
            if dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(0x55)
            junk.append(t)
    return junk


def test_control_the_allocator_reuses_a_freed_block_at_once():
    t = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    ptr = t.data_ptr()
    del t
    assert torch.empty(1 << 20, dtype=torch.float32, device="cuda").data_ptr() == ptr


def test_unfused_workspace_and_output_on_a_side_stream(recorded):
    x = inputs.make_inputs(1 << 22, 64, "nf4", 0.03, seed=71)
    dev = dq4.to_device(x)
    want = oracle_bits(x, "f16")
    side = torch.cuda.Stream()
    kw = dict(offset=float(x.offset), n=x.n, blocksize=64, out_dtype=torch.float16, stream=side)
    dq4.dq4_nested_dequant_unfused(**dev, **kw)     # the side stream's first use
    torch.cuda.synchronize()
    recorded.clear()
    keep = busy(side)
    y = dq4.dq4_nested_dequant_unfused(**dev, **kw)
    junk = scribble_and_check(recorded, side)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(y), want, "unfused on a side stream")
    del keep, junk


@pytest.mark.parametrize("route", ["rows", "fused"])
def test_out_prod_workspace_on_a_side_stream(recorded, route):
    n_rows, n_cols, m = 20000, 384, 32
    x = inputs.make_inputs(n_rows * n_cols, 64, "nf4", 0.03, seed=72, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    sel = np.random.Generator(np.random.PCG64(72)).choice(n_rows, m, replace=False)
    b = np.zeros((n_rows, m), np.float32)
    b[sel, np.arange(m)] = 1.0
    src1 = torch.from_numpy(b).cuda()
    side = torch.cuda.Stream()
    kw = dict(offset=float(x.offset), n_rows=n_rows, n_cols=n_cols, blocksize=64, src1=src1)

    def call(**more):
        if route == "rows":
            # four row windows through a workspace the binding allocates
            return dq4.dq4_out_prod_rows(**dev, **kw, workspace_bytes=n_cols * 4 * 5000, **more)
        assert dq4.dq4_out_prod_fused_workspace_bytes(n_rows, n_cols, m) > 0
        return dq4.dq4_out_prod_fused(**dev, **kw, **more)

    # a first call outside the test: it creates the library GEMM's handle (a
    # synchronizing step) and the side stream's first use
    call(stream=side)
    torch.cuda.synchronize()
    recorded.clear()
    keep = busy(side)
    y = call(stream=side)
    junk = scribble_and_check(recorded, side)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = weight_rows(x, n_cols, sel)
    assert (got == want).all(), f"{route}: selection out_prod differs from the weight rows"
    say(f"out_prod {route} on a side stream: exact")
    del keep, junk


def test_dequant_linear_weight_workspace_on_a_side_stream(recorded):
    """The weight workspace of dequantize-plus-linear; the result is checked
    through a selection: G has one 1 per row, so grad_a's row i is the FP16
    weight row it selects, summed with exact zeros in FP32 and rounded back
    to FP16 -- the same value (compared as values: a zero product may carry
    either sign into the sum)."""
    n_out, n_in, m = 512, 1024, 8
    x = inputs.make_inputs(n_out * n_in, 64, "nf4", 0.03, seed=73, n_rows=n_out, n_cols=n_in)
    dev = dq4.to_device(x)
    w16 = oracle_bits(x, "f16").reshape(n_out, n_in)
    sel = np.random.Generator(np.random.PCG64(73)).choice(n_out, m, replace=False)
    g = np.zeros((m, n_out), np.float16)
    g[np.arange(m), sel] = 1.0
    side = torch.cuda.Stream()
    gx = torch.from_numpy(g).cuda()

    def call():
        return dq4.dq4_dequant_linear(**dev, offset=float(x.offset), n_out=n_out, n_in=n_in,
                                      blocksize=64, x=gx, op="grad_a", stream=side)

    call()               # the GEMM handle and the side stream's first use, as above
    torch.cuda.synchronize()
    recorded.clear()
    keep = busy(side)
    y = call()
    junk = scribble_and_check(recorded, side)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    want = w16[sel].view(np.float16).astype(np.float32)
    assert (got == want).all(), "grad_a selection on a side stream differs from the weight rows"
    del keep, junk
