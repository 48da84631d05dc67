"""MFMA-tile order of E4M3 weight codes in the CPU oracle — test
infrastructure.

The grouped few-token call reads each Linear's weight codes in a tile order
of the library's own (the pages fix the codes and their per-channel scales,
not where the bytes sit in memory).  The order, as the library's header
states it: for row block rb (16 rows), K block i (128 bytes), half h in
{0, 1}, lane l in [0, 64) and byte e in [0, 16),

    tiled[(rb * (k / 128) + i) * 2048 + h * 1024 + 16 * l + e]
        = qw[16 * rb + (l % 16), 128 * i + 64 * h + 16 * (l // 16) + e]

so that each 16-row x 128-byte block is one contiguous 2 KB tile and the
tiles of a row block follow each other in K order.  Here it is written as
the reshape and axis order it amounts to: qw viewed as
[rb, r, i, h, g, e] (row 16 rb + r, K byte 128 i + 64 h + 16 g + e) is
stored in the order [rb, i, h, g, r, e] (lane l = r + 16 g).
"""

import numpy as np


def tile_weights_ref(qw: np.ndarray) -> np.ndarray:
    """Row-major E4M3 codes [n, k] (n % 16 == 0, k % 128 == 0) -> the same
    n * k bytes in tile order, as a flat uint8 array."""
    qw = np.asarray(qw, dtype=np.uint8)
    n, k = qw.shape
    if n % 16 or k % 128:
        raise ValueError("n must be a multiple of 16 and k of 128")
    view = qw.reshape(n // 16, 16, k // 128, 2, 4, 16)     # rb, r, i, h, g, e
    return np.ascontiguousarray(view.transpose(0, 2, 3, 4, 1, 5)).reshape(-1)
