"""GPU parity of the LLM.int8 correction-operand preparation (dq4_int8_prep).

bitsandbytes issue "Fuse LLM.int8 correction operand preparation into one
CUDA kernel", section "Exact correctness oracle": both outputs must match the
oracle bit for bit.  The cases follow what that section wants covered -- all
256 int8 codes; row scales that are zero, tiny, ordinary and huge; several
outlier counts; column sets in different orders, with repeats -- and the
empty-outlier call, which must launch nothing.  Shapes come from the issue's
benchmark plan (M from 1 to 2048; K and N from 3584 to 14336).  The call is
also captured in a HIP graph and replayed, since the binding no longer
synchronizes by default.
"""
from __future__ import annotations

import numpy as np
import pytest

import block_wise_bit_amd as dq4
import oracle
from gpu_util import assert_bits_equal, say

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

SPECIAL_SCB = [0.0, 2.0 ** -149, 2.0 ** -126, 1.0, 127.0, 65504.0 * 127, 3.4028234663852886e38]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from libs import ensure_hip_library
    ensure_hip_library()


def make_case(M, K, N, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    A = rng.integers(0, 1 << 16, size=(M, K), dtype=np.uint64).astype(np.uint16)  # any bits
    CB = rng.integers(-128, 128, size=(N, K), dtype=np.int64).astype(np.int8)
    SCB = np.exp(rng.normal(0.0, 3.0, N)).astype(np.float32)
    SCB[: len(SPECIAL_SCB)] = np.array(SPECIAL_SCB, np.float32)[: N]
    return A, CB, SCB


def column_sets(K, rng):
    return {
        "first": np.array([0]),
        "last": np.array([K - 1]),
        "pair": np.array([K - 1, 0]),
        "noncontiguous5": np.array([7, 3, K // 2, K - 2, 1]),
        "sorted16": np.sort(rng.choice(K, 16, replace=False)),
        "repeated64": rng.choice(K, 64, replace=True),
    }


def run(A, CB, SCB, cols):
    dA = torch.from_numpy(A.view(np.int16)).view(torch.float16).cuda()
    subA, subB = dq4.dq4_int8_prep(dA, torch.from_numpy(CB).cuda(), torch.from_numpy(SCB).cuda(),
                                   torch.from_numpy(cols.astype(np.int64)).cuda())
    return (subA.cpu().view(torch.int16).numpy().view(np.uint16),
            subB.cpu().view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("M", [1, 8, 64, 512, 2048])
@pytest.mark.parametrize("KN", [(3584, 3584), (4096, 4096), (8192, 8192), (14336, 14336),
                                (4096, 14336), (14336, 4096)])
def test_parity_grid(M, KN):
    K, N = KN
    A, CB, SCB = make_case(M, K, N, seed=M * 7 + K + N)
    rng = np.random.Generator(np.random.PCG64(M + K))
    for name, cols in column_sets(K, rng).items():
        say(f"int8 prep M={M} K={K} N={N} cols={name}")
        gA, gB = run(A, CB, SCB, cols)
        wA, wB = oracle.int8_prep(A, CB, SCB, cols)
        assert_bits_equal(gA.ravel(), wA.ravel(), f"subA {name}")
        assert_bits_equal(gB.ravel(), wB.ravel(), f"subB {name}")


def test_whole_code_domain_and_scale_kinds():
    """Every int8 code in every column position of rows whose scales cover
    zero, subnormal, normal, FP16-overflowing and the largest finite values."""
    codes = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    rng = np.random.Generator(np.random.PCG64(9))
    SCB = np.concatenate([np.array(SPECIAL_SCB, np.float32),
                          np.exp(rng.uniform(-30, 30, 249)).astype(np.float32)])
    CB = np.tile(codes, (SCB.size, 1))
    A = rng.integers(0, 1 << 16, size=(3, 256), dtype=np.uint64).astype(np.uint16)
    cols = np.arange(256)
    gA, gB = run(A, CB, SCB, cols)
    wA, wB = oracle.int8_prep(A, CB, SCB, cols)
    assert_bits_equal(gA.ravel(), wA.ravel(), "subA")
    assert_bits_equal(gB.ravel(), wB.ravel(), "subB")


def test_empty_outlier_path_launches_nothing_and_bad_indices_raise_on_request():
    A, CB, SCB = make_case(4, 64, 8, seed=1)
    dA = torch.from_numpy(A.view(np.int16)).view(torch.float16).cuda()
    dCB, dSCB = torch.from_numpy(CB).cuda(), torch.from_numpy(SCB).cuda()
    empty = torch.empty(0, dtype=torch.int64, device="cuda")
    subA, subB = dq4.dq4_int8_prep(dA, dCB, dSCB, empty)
    assert subA.shape == (4, 0) and subB.shape == (0, 8)
    for bad in ([64], [-1], [0, 64]):
        with pytest.raises(ValueError):
            dq4.dq4_int8_prep(dA, dCB, dSCB, torch.tensor(bad, dtype=torch.int64, device="cuda"),
                              validate=True)


def test_out_of_range_indices_without_validation_give_nan():
    """With the host check off (the default), the kernel reads nothing
    through an index outside [0, K) and writes FP16 NaN (0x7E00) to every
    output it feeds; the outputs of the valid indices still match the oracle."""
    M, K, N = 5, 64, 9
    A, CB, SCB = make_case(M, K, N, seed=2)
    cols = np.array([3, -1, 63, 64, 1 << 40, 0])
    good = np.array([c for c in range(cols.size) if 0 <= cols[c] < K])
    gA, gB = run(A, CB, SCB, cols)
    wA, wB = oracle.int8_prep(A, CB, SCB, cols[good])
    bad = np.setdiff1d(np.arange(cols.size), good)
    assert (gA[:, bad] == 0x7E00).all() and (gB[bad, :] == 0x7E00).all()
    assert_bits_equal(gA[:, good].ravel(), wA.ravel(), "subA, valid columns")
    assert_bits_equal(gB[good, :].ravel(), wB.ravel(), "subB, valid columns")


def test_graph_capture_replays_bit_exact():
    """The call captured in a HIP graph and replayed four times, with new A,
    CB, SCB and column values written eagerly (in place) between replays:
    every replay matches the oracle on the values of its own inputs."""
    M, K, N, L = 64, 4096, 4096, 16
    dA = torch.empty((M, K), dtype=torch.float16, device="cuda")
    dCB = torch.empty((N, K), dtype=torch.int8, device="cuda")
    dSCB = torch.empty(N, dtype=torch.float32, device="cuda")
    dcols = torch.empty(L, dtype=torch.int64, device="cuda")
    subA = torch.empty((M, L), dtype=torch.float16, device="cuda")
    subB = torch.empty((L, N), dtype=torch.float16, device="cuda")

    def fill(seed):
        A, CB, SCB = make_case(M, K, N, seed=seed)
        cols = np.random.Generator(np.random.PCG64(seed)).choice(K, L, replace=True)
        dA.copy_(torch.from_numpy(A.view(np.int16)).view(torch.float16))
        dCB.copy_(torch.from_numpy(CB))
        dSCB.copy_(torch.from_numpy(SCB))
        dcols.copy_(torch.from_numpy(cols.astype(np.int64)))
        return A, CB, SCB, cols

    fill(100)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the first call outside capture
        dq4.dq4_int8_prep(dA, dCB, dSCB, dcols, subA=subA, subB=subB)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dq4.dq4_int8_prep(dA, dCB, dSCB, dcols, subA=subA, subB=subB)
    for rep in range(4):
        A, CB, SCB, cols = fill(101 + rep)
        subA.fill_(0.0)
        subB.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        wA, wB = oracle.int8_prep(A, CB, SCB, cols)
        assert_bits_equal(subA.cpu().view(torch.int16).numpy().view(np.uint16).ravel(),
                          wA.ravel(), f"subA replay {rep}")
        assert_bits_equal(subB.cpu().view(torch.int16).numpy().view(np.uint16).ravel(),
                          wB.ravel(), f"subB replay {rep}")
