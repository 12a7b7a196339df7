"""The general vector path's index arithmetic, restated on the CPU (no GPU).

dq4_shift_tile_kernel aligns its tiles to the output's 128-byte lines, so a
unit's nibbles may start anywhere in the packed bytes and a unit may straddle
two outer blocks.  This test restates in numpy the launcher's routing (the
head, the full tiles, the tile order, the split point kK0 and the whole-unit
case) and the kernel's per-unit arithmetic (the packed dword or dwords a unit
reads through its buffer resource, the funnel shift, the block of each
element), and checks on seeded layouts of both unit sizes that every element
of the window is produced exactly once, from its own nibble, with its own
block's scale, into its own output slot.  A restatement can drift from the
kernel; the GPU parity tests are the ground truth, this pins the reasoning.
"""
from __future__ import annotations

import numpy as np
import pytest

THREADS, TILE = 256, 4096


def tile_units(out_f32: bool):
    """Unit index of each (unit slot u, lane t): FP16/BF16 u * 256 + t, FP32
    wave-contiguous runs of 64."""
    k_units = 4 if out_f32 else 2
    u, t = np.meshgrid(np.arange(k_units), np.arange(THREADS), indexing="ij")
    if not out_f32:
        return (u * 256 + t).ravel()
    return ((((t >> 6) * k_units + u) << 6) + (t & 63)).ravel()


def paired(slot: int, s: int) -> int:
    group = slot & ~((8 << s) - 1)
    x = slot - group
    return group | ((x % 8) << s) | (x // 8)


def check_layout(rng, n_total, e0, count, lb, p_off, out_shift, out_f32):
    E = 4 if out_f32 else 8
    ob = 4 if out_f32 else 2
    nbytes = (n_total + 1) // 2
    packed = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
    # the bytes as the kernel's buffer resource sees them: from the 4-byte
    # aligned address at or below `packed`, p_off & 3 bytes earlier
    pre = p_off & 3
    span = pre + ((e0 + count - 1) >> 1) + 1
    n_records = (span + 3) & ~3
    image = np.zeros(n_records + 8, np.uint8)
    image[pre:pre + nbytes] = packed[:max(0, min(nbytes, n_records - pre))]
    dwords = image[: n_records].view("<u4").astype(np.uint64)

    def load(byte):
        out = np.zeros(byte.shape, np.uint64)
        ok = byte + 4 <= n_records
        out[ok] = dwords[byte[ok] >> 2]
        return out

    # the launcher
    out_addr = out_shift * ob
    head = ((128 - out_addr % 128) % 128) // ob
    assert count >= TILE + 128
    n_full = (count - head) // TILE
    e_first = e0 + head
    sh = (pre * 8 + 4 * e_first) & 31
    k0 = E - e_first % E
    kk = 0 if sh % (4 * E) == 0 and k0 == E else k0      # the instantiation
    log2_share = min(lb - 5, 3)
    n_paired = 0 if out_f32 else n_full & ~((8 << log2_share) - 1)
    tiles = [paired(fs, log2_share) if fs < n_paired else fs for fs in range(n_full)]
    assert sorted(tiles) == list(range(n_full))

    covered = np.zeros(count, np.int64)
    covered[:head] += 1                               # slot 0, element by element
    covered[head + n_full * TILE:] += 1
    ul = tile_units(out_f32).astype(np.int64)
    for tile in tiles:
        e_tile = e0 + head + tile * TILE
        assert (out_addr + (head + tile * TILE) * ob) % 128 == 0   # 128-byte aligned stores
        bit0 = pre * 8 + 4 * e_tile
        assert (bit0 & 31) == sh                      # the same bit offset in every tile
        bit = bit0 + 4 * E * ul
        byte = (bit >> 5) << 2
        assert (byte >= 0).all() and (byte + 8 < (1 << 31)).all()
        lo = load(byte)
        ush = (sh + 4 * E * ul) & 31
        if kk == 0:
            assert (ush + 4 * E <= 32).all()          # the unit lies in one dword
            word = lo >> ush.astype(np.uint64)
        else:
            hi = load(byte + 4) if sh != 0 else np.zeros_like(lo)
            word = ((hi << np.uint64(32)) | lo) >> ush.astype(np.uint64)
        b0 = e_tile >> lb
        r = e_tile - (b0 << lb)
        first = r + ul * E
        for e in range(E):
            g = e_tile + ul * E + e
            nib = (word >> np.uint64(4 * e)) & np.uint64(15)
            want = (packed[g >> 1] >> (4 * (g & 1))) & 15
            assert np.array_equal(nib.astype(np.int64), want.astype(np.int64))
            if kk == 0:
                chosen = first >> lb
            else:
                chosen = ((first + E - 1) >> lb) if e >= kk else (first >> lb)
            assert np.array_equal(b0 + chosen, g >> lb)   # the element's own block
            j = g - e0
            assert ((j >= 0) & (j < count)).all()
            assert np.array_equal(ul * E + e, j - head - tile * TILE)   # its output slot
            np.add.at(covered, j, 1)
    assert (covered == 1).all()
    return kk


def layouts():
    rng = np.random.Generator(np.random.PCG64(20261204))
    cases = []
    for out_f32 in (False, True):
        E, ob = (4, 4) if out_f32 else (8, 2)
        # every split point and the whole-unit case, then random layouts
        for out_shift in range(0, 128 // ob):
            cases.append((out_f32, 0, out_shift, int(rng.integers(0, 4)), 6))
        for _ in range(12):
            cases.append((out_f32, int(rng.integers(0, 3000)), int(rng.integers(0, 128 // ob)),
                          int(rng.integers(0, 128)), int(rng.integers(5, 13))))
    return cases


@pytest.mark.parametrize("out_f32,e0,out_shift,p_off,lb", layouts())
def test_general_path_covers_every_element_once(out_f32, e0, out_shift, p_off, lb):
    rng = np.random.Generator(np.random.PCG64(e0 * 131 + out_shift * 7 + p_off + lb))
    count = 3 * TILE + 1000 + (e0 % 97)
    check_layout(rng, e0 + count, e0, count, lb, p_off, out_shift, out_f32)


def test_every_instantiation_is_reached():
    """Over the structured layouts, the routing reaches kK0 = 0 .. E for both unit sizes."""
    seen = {False: set(), True: set()}
    for out_f32, e0, out_shift, p_off, lb in layouts():
        rng = np.random.Generator(np.random.PCG64(1))
        count = 3 * TILE + 1000 + (e0 % 97)
        seen[out_f32].add(check_layout(rng, e0 + count, e0, count, lb, p_off, out_shift,
                                       out_f32))
    assert seen[False] == set(range(9))
    assert seen[True] == set(range(5))
