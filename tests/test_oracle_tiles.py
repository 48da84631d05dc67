"""Pins of oracle.tile_weights_ref (the MFMA-tile order of weight codes read
by the grouped few-token call), against byte positions derived by hand from
the layout (K panels of four 128-byte blocks, each panel holding every row
block's tiles for its K range), and structural properties that hold for any
permutation."""

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(11)


def _codes(n, k):
    return RNG.integers(0, 256, size=(n, k), dtype=np.uint8)


def test_hand_derived_positions_one_tile():
    """n = 16, k = 128: one 2 KB tile.  Worked by hand from the layout:
    lane 0 of half 0 is row 0, bytes 0..15; lane 1 is row 1 (lanes step
    through the 16 rows first); lane 16 is row 0 again, bytes 16..31; lane
    63 is row 15, bytes 48..63; half 1 starts over at K byte 64."""
    qw = _codes(16, 128)
    t = oracle.tile_weights_ref(qw)
    assert t.shape == (2048,)
    assert np.array_equal(t[0:16], qw[0, 0:16])
    assert np.array_equal(t[16:32], qw[1, 0:16])
    assert np.array_equal(t[15 * 16:16 * 16], qw[15, 0:16])
    assert np.array_equal(t[256:272], qw[0, 16:32])
    assert np.array_equal(t[1008:1024], qw[15, 48:64])
    assert np.array_equal(t[1024:1040], qw[0, 64:80])
    assert np.array_equal(t[2032:2048], qw[15, 112:128])


def test_hand_derived_positions_across_tiles():
    """n = 32, k = 256: tiles in the order (row block 0, K block 0),
    (0, 1), (1, 0), (1, 1), 2 KB each."""
    qw = _codes(32, 256)
    t = oracle.tile_weights_ref(qw)
    assert np.array_equal(t[2048:2064], qw[0, 128:144])       # (0, 1): row 0
    assert np.array_equal(t[4096:4112], qw[16, 0:16])         # (1, 0): row 16
    assert np.array_equal(t[4096 + 16:4096 + 32], qw[17, 0:16])
    assert np.array_equal(t[6144 + 1024 + 16 * 35:6144 + 1024 + 16 * 36],
                          qw[16 + 3, 128 + 64 + 32:128 + 64 + 48])   # lane 35: r 3, g 2


def test_hand_derived_positions_across_panels():
    """n = 32, k = 640: five K blocks, so panel 0 holds blocks 0-3 of both
    row blocks (32 x 512 = 16384 bytes: row block 0's four tiles, then row
    block 1's) and panel 1, from byte 16384, holds block 4 only (ipp = 1):
    row block 0's tile, then row block 1's."""
    qw = _codes(32, 640)
    t = oracle.tile_weights_ref(qw)
    assert t.shape == (32 * 640,)
    assert np.array_equal(t[3 * 2048:3 * 2048 + 16], qw[0, 384:400])      # rb 0, block 3
    assert np.array_equal(t[4 * 2048:4 * 2048 + 16], qw[16, 0:16])        # rb 1, block 0
    assert np.array_equal(t[5 * 2048:5 * 2048 + 16], qw[16, 128:144])     # rb 1, block 1
    assert np.array_equal(t[16384:16400], qw[0, 512:528])                 # panel 1, rb 0
    assert np.array_equal(t[16384 + 16 * 17:16384 + 16 * 18], qw[1, 528:544])  # lane 17
    assert np.array_equal(t[16384 + 2048:16384 + 2064], qw[16, 512:528])  # panel 1, rb 1
    assert np.array_equal(t[-16:], qw[31, 624:640])                       # last lane, h 1


def test_whole_panels_are_contiguous_k_slices():
    """Structure of the panel order: the first n * 512 bytes are a
    permutation of qw[:, :512] alone, the next n * 512 of qw[:, 512:1024]."""
    n, k = 48, 1280
    qw = _codes(n, k)
    t = oracle.tile_weights_ref(qw)
    for p in range(2):
        part = t[p * n * 512:(p + 1) * n * 512]
        assert np.array_equal(np.sort(part), np.sort(qw[:, p * 512:(p + 1) * 512].reshape(-1)))
    assert np.array_equal(np.sort(t[2 * n * 512:]), np.sort(qw[:, 1024:].reshape(-1)))


def test_is_a_permutation_of_distinct_rows():
    """Every (row, 16-byte chunk) lands in exactly one 16-byte slot of the
    output: mark each chunk with its own id in its first two bytes (k = 1408:
    panels of 4, 4 and 3 K blocks)."""
    n, k = 48, 1408
    qw = np.zeros((n, k), np.uint8)
    ids = np.arange(n * k // 16)
    chunks = qw.reshape(n, k // 16, 16)
    chunks[:, :, 0] = (ids.reshape(n, k // 16) & 0xFF)
    chunks[:, :, 1] = (ids.reshape(n, k // 16) >> 8)
    t = oracle.tile_weights_ref(qw).reshape(-1, 16)
    got = t[:, 0].astype(np.int64) | (t[:, 1].astype(np.int64) << 8)
    assert np.array_equal(np.sort(got), ids)
    assert np.all(t[:, 2:] == 0)


def test_rejects_ragged_shapes():
    with pytest.raises(ValueError):
        oracle.tile_weights_ref(_codes(24, 128))
    with pytest.raises(ValueError):
        oracle.tile_weights_ref(_codes(16, 192))
