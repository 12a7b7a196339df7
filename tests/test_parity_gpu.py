"""GPU parity: the HIP path against the CPU oracle, bit for bit (0 ULP).

The tolerance is zero for FP32, FP16 and BF16 alike: the FP32 operation order
is fixed (bitsandbytes issue "Fuse nested scale reconstruction into SM103
4-bit dequantization", section "Correctness requirements": bitwise identical
results), so any difference is a defect.  Every call goes through the C ABI
(libdq4.so) via the Python binding.
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from block_wise_bit_amd import inputs
from gpu_util import assert_bits_equal, bits_of, gpu_bits, oracle_bits, say, torch_dtype
from libs import ensure_hip_library

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

OFFSETS = (-0.1, -0.02, 0.0, 0.03, 0.1)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_hip_library()
    name = torch.cuda.get_device_properties(0).gcnArchName
    say(f"device: {torch.cuda.get_device_name(0)} arch {name}")
    return torch.device("cuda", 0)


def _check(x, dt, what):
    say(f"{what}: n={x.n} bs={x.blocksize} fmt={x.fmt} dt={dt} off={x.offset} seed={x.seed}")
    got = gpu_bits(x, dt)
    torch.cuda.synchronize()
    want = oracle_bits(x, dt)
    assert_bits_equal(got, want, what)


# ----------------------------------------------------------------------------
# every scale code x every 4-bit code, tails, partial blocks and groups
# ----------------------------------------------------------------------------
def structured(blocksize, fmt, offset):
    """Every scale code and every 4-bit code in both nibble positions, 2 full
    nested groups + a partial third (see tests/test_oracle_pins.py)."""
    nb = 2 * 256 + 3
    n = nb * blocksize
    j = np.arange(n // 2) % (blocksize // 2)
    packed = ((j % 16) | ((15 - j % 16) << 4)).astype(np.uint8)
    codes = (np.arange(nb) % 256).astype(np.uint8)
    rng = np.random.Generator(np.random.PCG64(7))
    scb = np.sort(inputs._uniform_pm1(rng, 256)).astype(np.float32)
    cb4 = inputs.nf4_style_codebook(rng) if fmt == "nf4" else inputs.fp4_style_codebook()
    absmax = np.array([np.exp(-3.0 + 0.5 * rng.standard_normal()), 0.125, 1.0], np.float32)
    return inputs.NestedInputs(packed, codes, absmax, scb, cb4, np.float32(offset), n, blocksize,
                               fmt=fmt)


@pytest.mark.parametrize("fmt", ["nf4", "fp4"])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("blocksize", [32, 64, 4096])
def test_every_scale_code_and_4bit_code(fmt, dt, blocksize):
    for off in OFFSETS:
        _check(structured(blocksize, fmt, off), dt, "all-codes")


@pytest.mark.parametrize("blocksize", inputs.TAIL_SWEEP_BLOCKSIZES)
def test_tails_partial_blocks_and_groups(blocksize):
    B = blocksize
    lengths = [1, 2, 3, 7, 8, 9, B - 1, B, B + 1, 4095, 4096, 4097, 8191, 8192, 8193, 16385,
               32769, 256 * B - 1, 256 * B,
               256 * B + 1, 256 * B + B + 1, 2 * 256 * B + 3 * B + 17]
    for n in lengths:
        for dt in ("f16", "f32", "bf16"):
            x = inputs.make_inputs(n, B, "fp4" if n % 2 else "nf4", -0.1 if n % 3 else 0.1,
                                   seed=1000 + n)
            _check(x, dt, f"tail n={n}")


def test_output_is_not_written_past_n():
    """Canaries after `out`: elements past n keep their values, on the vector
    path (aligned) and the per-element path (misaligned), for every dtype."""
    for n in (1, 13, 4095, 4096 + 5, 8192 + 5, 3 * 4096 + 1):
        for dt in ("f32", "f16", "bf16"):
            x = inputs.make_inputs(n, 32, "nf4", 0.03, seed=n)
            dev = dq4.to_device(x)
            guard = 300
            buf = torch.full((n + guard + 8,), 7.0, dtype=torch_dtype(dt), device="cuda")
            for shift in (0, 1):
                out = buf[shift: shift + n + guard]
                out.fill_(7.0)
                dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=n, blocksize=32,
                                       out_dtype=torch_dtype(dt), out=out)
                got = bits_of(out)
                assert_bits_equal(got[:n], oracle_bits(x, dt), f"canary n={n} {dt} shift={shift}")
                assert (out[n:].cpu() == 7.0).all(), f"wrote past n={n} ({dt}, shift={shift})"


def test_unaligned_pointers_give_the_same_bits():
    """Packed bytes and output one byte / one element off their alignment: the
    general vector path (funnel-shifted packed words, output-aligned tiles)
    gives the oracle's bits."""
    n = 100_003
    x = inputs.make_inputs(n, 64, "nf4", 0.03, seed=77)
    want = oracle_bits(x, "f16")
    dev = dq4.to_device(x)
    raw = torch.empty(x.packed.size + 1, dtype=torch.uint8, device="cuda")
    raw[1:].copy_(dev["packed"])
    dev_unaligned = dict(dev, packed=raw[1:])
    out = torch.empty(n + 1, dtype=torch.float16, device="cuda")[1:]
    y = dq4.dq4_nested_dequant(**dev_unaligned, offset=float(x.offset), n=n, blocksize=64,
                               out_dtype=torch.float16, out=out)
    assert_bits_equal(bits_of(y), want, "unaligned")


# ----------------------------------------------------------------------------
# conversion edges through the kernel: exact products, ties, subnormals, overflow
# ----------------------------------------------------------------------------
def test_conversion_edges_through_the_kernel():
    """scale_codebook = powers of two, absmax = 1, offset = 0 makes every block
    scale an exact power of two, so value = codebook4[k] * 2^e: 4096 chosen
    binary32 values per call reach the FP16/BF16 conversion, covering ties
    at both widths, FP16 subnormals and overflow, and FP32 subnormals."""
    rng = np.random.Generator(np.random.PCG64(99))
    B = 32
    nb = 256
    n = nb * B
    j = np.arange(n // 2) % (B // 2)
    packed = (j % 16 | ((15 - j % 16) << 4)).astype(np.uint8)
    codes = np.arange(nb, dtype=np.uint8)
    scb = (2.0 ** (np.arange(256) - 140.0)).astype(np.float32)   # 2^-140 .. 2^115
    absmax = np.ones(1, np.float32)
    lows = np.array([0x0FFF, 0x1000, 0x1001, 0x3000, 0x7FFF, 0x8000, 0x8001, 0x18000], np.uint32)
    for call in range(48):
        hi = rng.integers(0, 1 << 23, size=16, dtype=np.uint64).astype(np.uint32)
        low = lows[rng.integers(0, lows.size, size=16)]
        mant = (hi & ~np.uint32(0x1FFFF)) | low
        if call % 3 == 0:
            mant = hi
        sign = (rng.integers(0, 2, size=16).astype(np.uint32) << 31)
        cb4 = (sign | np.uint32(127 << 23) | (mant & np.uint32(0x7FFFFF))).view(np.float32)
        x = inputs.NestedInputs(packed, codes, absmax, scb, cb4, np.float32(0.0), n, B)
        for dt in ("f16", "bf16", "f32"):
            got = gpu_bits(x, dt)
            assert_bits_equal(got, oracle_bits(x, dt, threads=1), f"conversion call {call} {dt}")


def test_zero_and_negative_scales():
    """Offsets that cancel a block's product exactly (scale +0) and negative
    scales: signed zeros and signs follow IEEE rules, bit for bit."""
    B = 64
    nb = 512
    n = nb * B
    rng = np.random.Generator(np.random.PCG64(5))
    x = inputs.make_inputs(n, B, "fp4", 0.0, seed=5)
    x.scale_codebook = np.full(256, 0.5, np.float32)
    x.scale_codebook[::2] = -0.25
    x.nested_absmax = np.array([0.25, 2.0 ** -3], np.float32)
    for off in (0.125, -0.0625, 0.0, -0.0):
        x.offset = np.float32(off)
        for dt in ("f32", "f16", "bf16"):
            got = gpu_bits(x, dt)
            assert_bits_equal(got, oracle_bits(x, dt), f"zero/neg scale off={off} {dt}")
    del rng


# ----------------------------------------------------------------------------
# the workloads at full size
# ----------------------------------------------------------------------------
def test_square_4096_f32():
    wl = inputs.SQUARE_4096_F32
    _check(wl.inputs(), wl.out_dtype, wl.name)


@pytest.mark.parametrize("wl", inputs.mid_matrix_workloads(), ids=lambda w: w.name)
def test_mid_matrix(wl):
    _check(wl.inputs(), wl.out_dtype, wl.name)


def test_headline_28672x8192_f16():
    """The benchmarked call, in the benchmark's launch configuration, compared
    element by element with the oracle over the whole tensor."""
    wl = inputs.HEADLINE
    _check(wl.inputs(), wl.out_dtype, wl.name)


@pytest.mark.parametrize("wl", inputs.tail_sweep_workloads(), ids=lambda w: w.name)
def test_blocksize_tail_sweep(wl):
    _check(wl.inputs(), wl.out_dtype, wl.name)


def test_output_head_row_windows():
    """151936 x 5376 NF4 weight, F32 windows of <= 256 MiB (12483 rows, 13
    windows, the last 2140 rows) written into one reused buffer; each window
    equals the oracle's rows."""
    wl = inputs.OUTPUT_HEAD
    x = wl.inputs()
    dev = dq4.to_device(x)
    windows = dq4.dq4_row_windows(wl.n_rows, wl.n_cols, 4, dq4.ROW_BLOCK_BUDGET_BYTES)
    assert len(windows) == 13 and windows[0][1] == 12483 and windows[-1][1] == 2140
    buf = torch.empty(windows[0][1] * wl.n_cols, dtype=torch.float32, device="cuda")
    assert buf.numel() * 4 <= dq4.ROW_BLOCK_BUDGET_BYTES
    for r0, rows in windows:
        say(f"window r0={r0} rows={rows}")
        y = dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=wl.n_rows,
                                        n_cols=wl.n_cols, r0=r0, rows=rows, blocksize=64,
                                        out_dtype=torch.float32, out=buf)
        got = bits_of(y[: rows * wl.n_cols])
        want = oracle_bits(x, "f32", first=r0 * wl.n_cols, count=rows * wl.n_cols)
        assert_bits_equal(got, want, f"window r0={r0}")


@pytest.mark.parametrize("n_rows,n_cols,B,dt", [(997, 37, 32, "f16"), (300, 1027, 64, "bf16"),
                                                (64, 4100, 4096, "f32"), (5000, 24, 32, "f16")])
def test_misaligned_row_windows(n_rows, n_cols, B, dt):
    """Windows starting mid-byte, mid-block or off the 8-element grid take the
    per-element path; they still equal the oracle and concatenate to the whole."""
    x = inputs.make_inputs(n_rows * n_cols, B, "nf4", -0.02, seed=n_cols, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    whole = gpu_bits(x, dt, dev)
    assert_bits_equal(whole, oracle_bits(x, dt), "whole")
    elem = 2 if dt != "f32" else 4
    for budget in (n_cols * elem * 3, n_cols * elem * 50 + 1):
        parts = []
        for r0, rows in dq4.dq4_row_windows(n_rows, n_cols, elem, budget):
            y = dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=n_rows,
                                            n_cols=n_cols, r0=r0, rows=rows, blocksize=B,
                                            out_dtype=torch_dtype(dt))
            parts.append(bits_of(y))
        assert_bits_equal(np.concatenate(parts), whole, f"windows budget={budget}")


# ----------------------------------------------------------------------------
# forms, streams, graphs, sizes
# ----------------------------------------------------------------------------
def test_allocating_and_out_forms_and_repeated_launches():
    x = inputs.make_inputs(1_000_003, 128, "nf4", 0.03, seed=8)
    dev = dq4.to_device(x)
    want = oracle_bits(x, "bf16")
    a = dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=128,
                               out_dtype=torch.bfloat16)
    out = torch.empty(x.n, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):
        b = dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=128,
                                   out_dtype=torch.bfloat16, out=out)
        assert b.data_ptr() == out.data_ptr()
        assert_bits_equal(bits_of(b), want, "out form")
    assert_bits_equal(bits_of(a), want, "allocating form")


def test_current_stream_ordering():
    """Inputs written by stream-ordered copies on a side stream, the kernel on
    the same stream, no host synchronization in between."""
    x = inputs.make_inputs(4_000_000, 64, "fp4", -0.02, seed=9)
    want = oracle_bits(x, "f16")
    s = torch.cuda.Stream()
    host = {k: torch.from_numpy(v).pin_memory() for k, v in
            dict(packed=x.packed, scale_codes=x.scale_codes, nested_absmax=x.nested_absmax,
                 scale_codebook=x.scale_codebook, codebook4=x.codebook4).items()}
    with torch.cuda.stream(s):
        dev = {k: torch.empty_like(v, device="cuda") for k, v in host.items()}
        for k in dev:
            dev[k].copy_(host[k], non_blocking=True)
        out = torch.empty(x.n, dtype=torch.float16, device="cuda")
        out.fill_(0)
        dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=64,
                               out_dtype=torch.float16, out=out)
        res = torch.empty(x.n, dtype=torch.float16, pin_memory=True)
        res.copy_(out, non_blocking=True)
    s.synchronize()
    assert_bits_equal(bits_of(res), want, "side stream")


def test_torch_style_wrapper_matches_the_c_named_calls():
    """nested_dequant: whole tensor and row window, allocating and in-place
    forms, give the bits of the C-named calls and of the oracle; bad
    arguments raise ValueError."""
    n_rows, n_cols = 123, 1000
    x = inputs.make_inputs(n_rows * n_cols, 128, "nf4", 0.1, seed=4242, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    whole = dq4.nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=128)
    assert whole.dtype == torch.float16
    assert_bits_equal(bits_of(whole), oracle_bits(x, "f16"), "wrapper whole")
    out = torch.empty(x.n, dtype=torch.bfloat16, device="cuda")
    same = dq4.nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=128,
                              dtype=torch.bfloat16, out=out)
    assert same.data_ptr() == out.data_ptr()
    assert_bits_equal(bits_of(out), oracle_bits(x, "bf16"), "wrapper .out")
    r0, count = 40, 51
    win = dq4.nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=128,
                             dtype=torch.float32, rows=(n_rows, n_cols, r0, count))
    ref = dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=n_rows,
                                      n_cols=n_cols, r0=r0, rows=count, blocksize=128,
                                      out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(win.view(torch.int32), ref.view(torch.int32))
    assert_bits_equal(bits_of(win), oracle_bits(x, "f32", r0 * n_cols, count * n_cols),
                      "wrapper rows")
    with pytest.raises(ValueError):
        dq4.nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=96)
    with pytest.raises(ValueError):
        dq4.nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=128,
                           rows=(n_rows, n_cols, 100, 24))


def test_graph_capture_replays():
    """One call captured in a HIP graph and replayed several times, with other
    eager work in between; every replay equals the eager result."""
    x = inputs.make_inputs(3_000_017, 64, "nf4", 0.03, seed=10)
    dev = dq4.to_device(x)
    want = oracle_bits(x, "f16")
    out = torch.empty(x.n, dtype=torch.float16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the path outside capture
        dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=64,
                               out_dtype=torch.float16, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=64,
                               out_dtype=torch.float16, out=out)
    for rep in range(4):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(bits_of(out), want, f"replay {rep}")
        junk = torch.randn(1 << 20, device="cuda") * 2  # unrelated eager work
        del junk


def test_beyond_2_pow_31_elements():
    """64-bit indexing: a 2^31 + 4099 element call (1 GiB packed, 4 GiB FP16
    out); sampled ranges at the start, around 2^31 and at the end equal the
    oracle's output for those global elements."""
    n = (1 << 31) + 4099
    B = 256
    x = inputs.make_inputs(n, B, "nf4", 0.1, seed=31)
    dev = dq4.to_device(x)
    y = dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=n, blocksize=B,
                               out_dtype=torch.float16)
    for first, count in ((0, 1 << 20), ((1 << 31) - (1 << 19), n - (1 << 31) + (1 << 19)),
                         (n - 5000, 5000), (1 << 30, 4096)):
        got = bits_of(y[first: first + count])
        assert_bits_equal(got, oracle_bits(x, "f16", first, count), f"range {first}+{count}")
    del y, dev
    torch.cuda.empty_cache()


def test_row_windows_past_2_pow_31_and_2_pow_32_elements():
    """64-bit indexing of the row-window call: a weight of 2^32 + 2^20
    elements (2 GiB packed, n_cols = 4096), windows straddling elements
    2^31 and 2^32, the weight's last rows, and a short window past 2^32
    that starts inside a nested group (rows 2^20 + 7 .. + 2; a group of 256
    blocks of 64 is 4 rows here), in FP16 and FP32; each equals the oracle's
    elements."""
    n_rows, n_cols = (1 << 20) + 256, 4096
    x = inputs.make_inputs(n_rows * n_cols, 64, "nf4", 0.02, seed=782, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    windows = [((1 << 19) - 150, 300),        # across element 2^31
               ((1 << 20) - 150, 300),        # across element 2^32
               (n_rows - 257, 257),           # the last rows
               ((1 << 20) + 7, 3)]            # a short window past 2^32
    for dt in ("f16", "f32"):
        for r0, rows in windows:
            say(f"window {dt} r0={r0} rows={rows}")
            y = dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=n_rows,
                                            n_cols=n_cols, r0=r0, rows=rows, blocksize=64,
                                            out_dtype=torch_dtype(dt))
            want = oracle_bits(x, dt, first=r0 * n_cols, count=rows * n_cols)
            assert_bits_equal(bits_of(y), want, f"window {dt} r0={r0} rows={rows}")
    del dev
    torch.cuda.empty_cache()


def test_bad_arguments_raise_and_write_nothing():
    x = inputs.make_inputs(1000, 64, "nf4", 0.03, seed=1)
    dev = dq4.to_device(x)
    out = torch.full((1000,), 3.0, dtype=torch.float16, device="cuda")
    for kwargs in (dict(blocksize=48), dict(blocksize=8192), dict(nested_blocksize=128)):
        args = dict(offset=0.03, n=1000, blocksize=64, out_dtype=torch.float16, out=out)
        args.update(kwargs)
        with pytest.raises(ValueError):
            dq4.dq4_nested_dequant(**dev, **args)
    with pytest.raises(ValueError):
        dq4.dq4_nested_dequant(**dict(dev, packed=dev["packed"][:10]), offset=0.0, n=1000,
                               blocksize=64, out=out)
    with pytest.raises(ValueError):
        dq4.dq4_nested_dequant_rows(**dev, offset=0.0, n_rows=10, n_cols=100, r0=5, rows=6,
                                    blocksize=64)
    torch.cuda.synchronize()
    assert (out.cpu() == 3.0).all()
    y = dq4.dq4_nested_dequant(**dev, offset=0.0, n=0, blocksize=64)
    assert y.numel() == 0


# ----------------------------------------------------------------------------
# the memory twin (a diagnostic with the FP16 call's traffic, no arithmetic)
# ----------------------------------------------------------------------------
def test_memory_twin_writes_each_packed_word_four_times():
    rng = np.random.Generator(np.random.PCG64(31))
    n = 4096 * 37
    packed = rng.integers(0, 256, size=n // 2, dtype=np.uint8)
    y = dq4.dq4_memory_twin_f16(torch.from_numpy(packed).cuda(), n)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int32).numpy().view(np.uint32)
    want = np.repeat(packed.view(np.uint32), 4)
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        dq4.dq4_memory_twin_f16(torch.from_numpy(packed).cuda(), n - 8)


# ----------------------------------------------------------------------------
# the shifted vector path: element-aligned but otherwise misaligned windows
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("bs", [32, 64, 4096])
@pytest.mark.parametrize("out_shift,packed_shift",
                         [(1, 0), (0, 1), (3, 2), (5, 3), (8, 0), (4, 0), (8, 4), (2, 0),
                          (6, 1), (7, 0)])
def test_shifted_vector_path(dt, bs, out_shift, packed_shift):
    """Outputs shifted by out_shift elements and packed bytes by packed_shift
    bytes from their natural alignment, over 5 full tiles plus a head and a
    tail: the funnel-shifted units and two-scale elements give the oracle's
    bits.  (8, 0) and (8, 4) take the whole-unit instantiation for every
    output type, (4, 0) for FP32 (units on half dwords), the rest the
    general one; over the shifts, every split point k0 = 1 .. E of a unit's
    elements between two blocks is taken for each output type."""
    n = 5 * 4096 + 1000 + 3
    x = inputs.make_inputs(n, bs, "nf4", -0.05, seed=77 + bs + out_shift)
    dev = dq4.to_device(x)
    if packed_shift:
        holder = torch.zeros(x.packed.size + packed_shift, dtype=torch.uint8, device="cuda")
        holder[packed_shift:] = dev["packed"]
        dev["packed"] = holder[packed_shift:]
    tdt = torch_dtype(dt)
    backing = torch.full((n + out_shift + 8,), float("nan"), dtype=tdt, device="cuda")
    out = backing[out_shift:out_shift + n]
    dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=n, blocksize=bs, out_dtype=tdt,
                           out=out)
    torch.cuda.synchronize()
    assert_bits_equal(bits_of(out), oracle_bits(x, dt), f"shifted {dt} bs={bs}")
    assert torch.isnan(backing[:out_shift].float()).all()
    assert torch.isnan(backing[out_shift + n:].float()).all()


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_odd_width_row_windows_full_size(dt):
    """A 28672 x 8191 weight (odd width: windows start mid-byte) in windows of
    4001 rows, every window against the oracle's rows."""
    n_rows, n_cols = 28672, 8191
    x = inputs.make_inputs(n_rows * n_cols, 64, "nf4", 0.03, seed=8191, n_rows=n_rows,
                           n_cols=n_cols)
    dev = dq4.to_device(x)
    tdt = torch_dtype(dt)
    buf = torch.empty(4001 * n_cols, dtype=tdt, device="cuda")
    for r0 in range(0, n_rows, 4001):
        rows = min(4001, n_rows - r0)
        say(f"odd-width window r0={r0} rows={rows} {dt}")
        y = dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=n_rows,
                                        n_cols=n_cols, r0=r0, rows=rows, blocksize=64,
                                        out_dtype=tdt, out=buf)
        got = bits_of(y[: rows * n_cols])
        want = oracle_bits(x, dt, first=r0 * n_cols, count=rows * n_cols)
        assert_bits_equal(got, want, f"odd-width window r0={r0}")
