"""GPU parity over a seeded random sweep of layouts, bit for bit (0 ULP).

The structured tests pin chosen layouts; this sweep draws 240 more from one
seed (and 36 from another, all of them layouts of the general vector path's
whole-unit instantiation): shapes (1..400 rows x 1..3000 columns), every block size 32..4096,
NF4/FP4, the three output types, offsets of both signs (and exact zero),
whole-tensor calls and row windows, with the packed bytes and the output
shifted off their natural alignment in some cases so that both the vector
path and the per-element path are exercised.  Each case prints its
parameters before it runs, and every output is compared with the oracle's
elements one by one (bitsandbytes issue "Fuse nested scale reconstruction
into SM103 4-bit dequantization", section "Correctness requirements").
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from block_wise_bit_amd import inputs
from gpu_util import assert_bits_equal, bits_of, oracle_bits, say, torch_dtype
from libs import ensure_hip_library

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

N_CASES = 240
BLOCKSIZES = (32, 64, 128, 256, 512, 1024, 2048, 4096)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_hip_library()


def _cases():
    rng = np.random.Generator(np.random.PCG64(20261202))
    for c in range(N_CASES):
        n_rows = int(rng.integers(1, 401))
        n_cols = int(rng.integers(1, 3001))
        bs = int(BLOCKSIZES[rng.integers(0, len(BLOCKSIZES))])
        fmt = ("nf4", "fp4")[int(rng.integers(0, 2))]
        dt = ("f16", "bf16", "f32")[int(rng.integers(0, 3))]
        pick = rng.random()
        offset = 0.0 if pick < 0.1 else float(np.float32(rng.uniform(-0.2, 0.2)))
        window = rng.random() < 0.5
        r0 = int(rng.integers(0, n_rows)) if window else 0
        rows = int(rng.integers(0, n_rows - r0 + 1)) if window else n_rows
        packed_shift = int(rng.integers(0, 4)) if rng.random() < 0.3 else 0
        out_shift = int(rng.integers(1, 8)) if rng.random() < 0.3 else 0
        yield (c, n_rows, n_cols, bs, fmt, dt, offset, window, r0, rows, packed_shift, out_shift)


def _whole_unit_cases():
    """Layouts the general vector path's whole-unit instantiation takes: the
    first full tile's 4-bit codes start on a packed dword (FP32: half of one)
    and its units inside one block.  n_cols is a multiple of 8, so every row
    window starts on a multiple of 8 elements; the output is 16 bytes (or, for
    FP32, 16 or 32 bytes) past a 128-byte line and the packed bytes 0 or 4
    bytes past a line."""
    rng = np.random.Generator(np.random.PCG64(20261203))
    for c in range(N_WHOLE_CASES):
        n_cols = 8 * int(rng.integers(8, 376))
        n_rows = int(rng.integers(-(-9000 // n_cols), 401))
        bs = int(BLOCKSIZES[rng.integers(0, len(BLOCKSIZES))])
        fmt = ("nf4", "fp4")[int(rng.integers(0, 2))]
        dt = ("f16", "bf16", "f32")[int(rng.integers(0, 3))]
        offset = float(np.float32(rng.uniform(-0.2, 0.2)))
        window = rng.random() < 0.5
        rows_min = -(-(4096 + 128) // n_cols)
        r0 = int(rng.integers(0, n_rows - rows_min + 1)) if window else 0
        rows = int(rng.integers(rows_min, n_rows - r0 + 1)) if window else n_rows
        packed_shift = int((0, 4)[rng.integers(0, 2)])
        out_shift = 8 if dt != "f32" else int((4, 8)[rng.integers(0, 2)])
        yield (c, n_rows, n_cols, bs, fmt, dt, offset, window, r0, rows, packed_shift, out_shift)


N_WHOLE_CASES = 36


@pytest.mark.parametrize("case", list(_whole_unit_cases()), ids=lambda c: f"whole{c[0]}")
def test_random_whole_unit_layout(case):
    _run_case(case)


@pytest.mark.parametrize("case", list(_cases()), ids=lambda c: f"case{c[0]}")
def test_random_layout(case):
    _run_case(case)


def _run_case(case):
    c, n_rows, n_cols, bs, fmt, dt, offset, window, r0, rows, packed_shift, out_shift = case
    n = n_rows * n_cols
    say(f"case {c}: {n_rows}x{n_cols} bs={bs} {fmt} {dt} offset={offset} "
        f"{'rows ' + str(r0) + '+' + str(rows) if window else 'whole'} "
        f"packed_shift={packed_shift} out_shift={out_shift}")
    x = inputs.make_inputs(n, bs, fmt, offset, seed=inputs.SEED_BASE + 1000 + c,
                           n_rows=n_rows, n_cols=n_cols)
    dev = dq4.to_device(x)
    if packed_shift:
        # the same bytes, starting packed_shift bytes into a larger buffer
        holder = torch.zeros(x.packed.size + packed_shift, dtype=torch.uint8, device="cuda")
        holder[packed_shift:] = dev["packed"]
        dev["packed"] = holder[packed_shift:]
    first, count = (r0 * n_cols, rows * n_cols) if window else (0, n)
    tdt = torch_dtype(dt)
    backing = torch.full((count + out_shift,), float("nan"), dtype=tdt, device="cuda")
    out = backing[out_shift:]
    if window:
        dq4.dq4_nested_dequant_rows(**dev, offset=float(x.offset), n_rows=n_rows, n_cols=n_cols,
                                    r0=r0, rows=rows, blocksize=bs, out_dtype=tdt, out=out)
    else:
        dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=n, blocksize=bs, out_dtype=tdt,
                               out=out)
    torch.cuda.synchronize()
    got = bits_of(out)
    want = oracle_bits(x, dt, first=first, count=count) if count else got[:0]
    assert_bits_equal(got, want, f"case {c}")
    # nothing before the output was touched
    if out_shift:
        assert torch.isnan(backing[:out_shift].float()).all(), f"case {c}: wrote before out"
