"""GPU checks of dequantize-plus-linear (dq4_dequant_linear).

bitsandbytes issue "Fuse nested scale reconstruction into SM103 4-bit
dequantization", sections "Problem" and "Correctness requirements": the
dequantize-plus-linear fallback and MatMul4Bit.backward's grad_A consume the
same nested dequantization, and that page allows the usual GEMM tolerances
for their outputs only once the dequantized weight has been shown to be
bitwise equal.  So each case first checks the dequantized weight bit for bit
against the oracle, then the GEMM against a float64 sum with a tolerance
derived from the arithmetic: FP16/BF16 products are exact in FP32, an FP32
sum of K of them is within gamma_K * S of the exact sum (gamma_K = K u /
(1 - K u), u = 2^-24, S = sum |x| |w|), and the final rounding to the output
type adds at most u_out * (|y| + gamma_K * S) plus half its smallest
subnormal (u_out = 2^-11 for FP16, 2^-8 for BF16).
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
from block_wise_bit_amd import inputs
from gpu_util import assert_bits_equal, bits_of, oracle_bits, say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24
OUT = {"f16": (torch.float16, 2.0 ** -11, 2.0 ** -25), "bf16": (torch.bfloat16, 2.0 ** -8, 2.0 ** -134)}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from libs import ensure_hip_library
    ensure_hip_library()


def _as_float64(bits16: np.ndarray, dt: str) -> np.ndarray:
    t = torch.from_numpy(bits16.view(np.int16)).view(OUT[dt][0])
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("op", ["forward", "grad_a"])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(4096, 11008, 512, "nf4"), (11008, 4096, 64, "fp4"),
                                   (1000, 37 * 64 + 8, 3, "nf4")])
def test_dequant_linear(op, dt, shape):
    n_out, n_in, m, fmt = shape
    tdt, u_out, sub = OUT[dt]
    x = inputs.make_inputs(n_out * n_in, 64, fmt, -0.02, seed=n_out + n_in, n_rows=n_out,
                           n_cols=n_in)
    dev = dq4.to_device(x)
    k = n_in if op == "forward" else n_out
    rng = np.random.Generator(np.random.PCG64(m))
    xin = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(tdt).cuda()
    ws = torch.empty(n_out * n_in, dtype=tdt, device="cuda")
    say(f"linear {op} {dt} W {n_out}x{n_in} m={m}")
    y = dq4.dq4_dequant_linear(
        **dev, offset=float(x.offset), n_out=n_out, n_in=n_in, blocksize=64, x=xin, op=op,
        w_workspace=ws)
    # 1. the dequantized weight, bit for bit
    w_bits = oracle_bits(x, dt)
    assert_bits_equal(bits_of(ws), w_bits, "dequantized weight")
    # 2. the GEMM, against a float64 sum
    w = _as_float64(w_bits, dt).reshape(n_out, n_in)
    xv = xin.cpu().to(torch.float64).numpy()
    if op == "forward":
        exact, s = xv @ w.T, np.abs(xv) @ np.abs(w).T
    else:
        exact, s = xv @ w, np.abs(xv) @ np.abs(w)
    gamma = k * U32 / (1 - k * U32)
    bound = u_out * (np.abs(exact) + gamma * s) + gamma * s + sub
    got = y.cpu().to(torch.float64).numpy()
    err = np.abs(got - exact)
    say(f"  max err {err.max():.3e}, worst err/bound {(err / bound).max():.3e}")
    assert np.isfinite(got).all()
    assert (err <= bound).all()


def test_linear_argument_errors():
    x = inputs.make_inputs(64 * 128, 64, "nf4", 0.0, seed=1, n_rows=64, n_cols=128)
    dev = dq4.to_device(x)
    xin = torch.zeros((4, 128), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        dq4.dq4_dequant_linear(**dev, offset=0.0, n_out=64, n_in=128, blocksize=64, x=xin,
                               op="backward")
    with pytest.raises(ValueError):
        dq4.dq4_dequant_linear(**dev, offset=0.0, n_out=64, n_in=128, blocksize=64,
                               x=xin.float(), op="forward")
    with pytest.raises(ValueError):   # grad_A wants x of width n_out
        dq4.dq4_dequant_linear(**dev, offset=0.0, n_out=64, n_in=128, blocksize=64, x=xin,
                               op="grad_a")
    y = dq4.dq4_dequant_linear(**dev, offset=0.0, n_out=64, n_in=128, blocksize=64,
                               x=torch.zeros((0, 128), dtype=torch.float16, device="cuda"))
    assert y.shape == (0, 64)
