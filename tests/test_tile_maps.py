"""The vector kernels' slot -> tile maps, restated on the CPU (no GPU).

Workgroups are dispatched to MI355X's 8 XCDs in turn (workgroup i to XCD
i mod 8).  dq4_tile_kernel runs the partial last tile, if any, in slot 0 and
the full tiles in slots 1 onward; for FP16/BF16 output it permutes each
aligned group of 8 * 2^s full-tile slots so that the 2^s tiles reading one
128-byte line of scale codes (block size 2^(s+5) and up) land on one XCD.
These checks pin that the maps are bijections onto the tiles and that the
pairing does what it is for.
"""
from __future__ import annotations

import pytest

XCDS = 8


def paired(slot: int, s: int) -> int:
    group = slot & ~((XCDS << s) - 1)
    x = slot - group
    return group | ((x % XCDS) << s) | (x // XCDS)


def tile_of_slot(slot: int, n_full: int, n_tiles: int, lb: int, stream: bool) -> int:
    edge = n_tiles - n_full
    if slot < edge:
        return n_full                                  # the partial tile
    fs = slot - edge
    s = min(lb - 5, 3)
    n_paired = n_full & ~((XCDS << s) - 1) if stream else 0
    return paired(fs, s) if fs < n_paired else fs


@pytest.mark.parametrize("count", [4096, 4097, 8191, 5 * 4096, 64 * 4096 + 1, 1000 * 4096 + 37])
@pytest.mark.parametrize("lb", [5, 6, 7, 8, 12])
@pytest.mark.parametrize("stream", [True, False])
def test_every_tile_once(count, lb, stream):
    n_full = count // 4096
    n_tiles = -(-count // 4096)
    tiles = [tile_of_slot(slot, n_full, n_tiles, lb, stream) for slot in range(n_tiles)]
    assert sorted(tiles) == list(range(n_tiles))
    if n_tiles > n_full:
        assert tiles[0] == n_full                      # the partial tile is dispatched first


@pytest.mark.parametrize("lb", [6, 7, 8, 12])
def test_tiles_sharing_a_code_line_share_an_xcd(lb):
    """A 4096-element tile covers 4096 / 2^lb codes, so 2^min(lb-5, 3) tiles
    read each 128-byte line of codes; within the paired slots they run on one
    XCD.  (Slot k of a launch with a partial tile is workgroup k + 1.)"""
    for edge in (0, 1):
        n_full = 40 * XCDS * 8
        s = min(lb - 5, 3)
        share = 1 << s
        xcd_of_tile = {}
        for slot in range(edge, n_full + edge):
            xcd_of_tile[tile_of_slot(slot, n_full, n_full + edge, lb, True)] = slot % XCDS
        for first in range(0, n_full, share):
            assert len({xcd_of_tile[t] for t in range(first, first + share)}) == 1


def test_unfused_value_kernel_map():
    """The unfused value kernel runs its partial tile in slot 0 too."""
    for count in (4096, 4097, 3 * 4096 + 5, 77 * 4096):
        n_full = count // 4096
        n_tiles = -(-count // 4096)
        edge = n_tiles - n_full
        tiles = [n_full if slot < edge else slot - edge for slot in range(n_tiles)]
        assert sorted(tiles) == list(range(n_tiles))
