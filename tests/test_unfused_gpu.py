"""GPU parity of the unfused three-launch baseline (dq4_nested_dequant_unfused).

The unfused sequence of the bitsandbytes issue "Fuse nested scale
reconstruction into SM103 4-bit dequantization" (section "Problem") must give
exactly the oracle's bits -- and therefore exactly the fused kernel's -- for
every output type, block size, tail and alignment (section "Correctness
requirements": bitwise identical, no tolerance).
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


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_hip_library()


def _unfused_bits(x, dt, dev=None, out=None, ws=None):
    dev = dev or dq4.to_device(x)
    y = dq4.dq4_nested_dequant_unfused(**dev, offset=float(x.offset), n=x.n,
                                       blocksize=x.blocksize, out_dtype=torch_dtype(dt), out=out,
                                       scale_workspace=ws)
    return bits_of(y[: x.n])


def _all_codes(blocksize, fmt, offset):
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


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("blocksize", [32, 4096])
def test_unfused_every_code_pair(dt, blocksize):
    for fmt in ("nf4", "fp4"):
        for off in (-0.1, 0.0, 0.03):
            x = _all_codes(blocksize, fmt, off)
            say(f"unfused all-codes bs={blocksize} {fmt} {dt} off={off}")
            assert_bits_equal(_unfused_bits(x, dt), oracle_bits(x, dt), "unfused all-codes")


@pytest.mark.parametrize("blocksize", [32, 64, 512, 4096])
def test_unfused_tails(blocksize):
    B = blocksize
    for n in (1, 3, B + 1, 8191, 8193, 256 * B + B + 1, 2 * 256 * B + 3 * B + 17):
        x = inputs.make_inputs(n, B, "fp4" if n % 2 else "nf4", -0.02, seed=2000 + n)
        for dt in ("f16", "f32"):
            assert_bits_equal(_unfused_bits(x, dt), oracle_bits(x, dt), f"unfused n={n} {dt}")


def test_unfused_equals_fused_on_the_headline_workload():
    wl = inputs.HEADLINE
    x = wl.inputs()
    dev = dq4.to_device(x)
    say(f"{wl.name}: fused vs unfused vs oracle")
    fused = bits_of(dq4.dq4_nested_dequant(**dev, offset=float(x.offset), n=x.n, blocksize=64,
                                           out_dtype=torch.float16))
    unfused = _unfused_bits(x, "f16", dev)
    assert_bits_equal(unfused, fused, "unfused vs fused")
    assert_bits_equal(unfused, oracle_bits(x, "f16"), "unfused vs oracle")


@pytest.mark.parametrize("wl", [w for w in inputs.mid_matrix_workloads() if w.n_rows == 11008],
                         ids=lambda w: w.name)
def test_unfused_mid_matrix(wl):
    x = wl.inputs()
    assert_bits_equal(_unfused_bits(x, wl.out_dtype), oracle_bits(x, wl.out_dtype), wl.name)


def test_unfused_unaligned_and_reused_workspace():
    """The per-element value pass (unaligned pointers), and one workspace
    reused by two calls of different sizes."""
    n = 100_003
    x = inputs.make_inputs(n, 64, "nf4", 0.03, seed=77)
    dev = dq4.to_device(x)
    raw = torch.empty(x.packed.size + 1, dtype=torch.uint8, device="cuda")
    raw[1:].copy_(dev["packed"])
    out = torch.empty(n + 1, dtype=torch.bfloat16, device="cuda")[1:]
    ws = torch.empty(dq4.dq4_unfused_workspace_bytes(n, 64) // 4, dtype=torch.float32,
                     device="cuda")
    y = dq4.dq4_nested_dequant_unfused(**dict(dev, packed=raw[1:]), offset=float(x.offset), n=n,
                                       blocksize=64, out_dtype=torch.bfloat16, out=out,
                                       scale_workspace=ws)
    assert_bits_equal(bits_of(y), oracle_bits(x, "bf16"), "unfused unaligned")
    small = inputs.make_inputs(5_000, 64, "fp4", -0.1, seed=78)
    assert_bits_equal(_unfused_bits(small, "f16", ws=ws), oracle_bits(small, "f16"),
                      "unfused reused workspace")
    with pytest.raises(ValueError):
        dq4.dq4_nested_dequant_unfused(**dev, offset=0.0, n=n, blocksize=64,
                                       scale_workspace=ws[:10])
