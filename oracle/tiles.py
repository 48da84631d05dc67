"""MFMA-tile order of E4M3 weight codes in the CPU oracle — test
infrastructure.

The grouped few-token call reads each Linear's weight codes in a tile order
of the library's own (the pages fix the codes and their per-channel scales,
not where the bytes sit in memory).  The order, as the library's header
states it: K is cut into panels of four 128-byte K blocks (512 bytes; the
last panel holds the k / 128 - 4 p blocks that are left, ipp(p) of them).
For panel p, row block rb (16 rows), block j of the panel (K block
i = 4 p + j), half h in {0, 1}, lane l in [0, 64) and byte e in [0, 16),

    tiled[p * n * 512 + (rb * ipp(p) + j) * 2048 + h * 1024 + 16 * l + e]
        = qw[16 * rb + (l % 16), 128 * i + 64 * h + 16 * (l // 16) + e]

so that each 16-row x 128-byte block is one contiguous 2 KB tile, a panel
holds the tiles of every row block for its 512 bytes of K (row block by
row block, K order inside), and the panels follow each other in K order.
Here each panel is written as the reshape and axis order it amounts to:
the panel's columns of qw viewed as [rb, r, j, h, g, e] (row 16 rb + r,
K byte 128 (4 p + j) + 64 h + 16 g + e) are stored in the order
[rb, j, h, g, r, e] (lane l = r + 16 g), and the panels are concatenated.
"""

import numpy as np

PANEL_BLOCKS = 4   # 128-byte K blocks per panel


def tile_weights_ref(qw: np.ndarray) -> np.ndarray:
    """Row-major E4M3 codes [n, k] (n % 16 == 0, k % 128 == 0) -> the same
    n * k bytes in tile order, as a flat uint8 array."""
    qw = np.asarray(qw, dtype=np.uint8)
    n, k = qw.shape
    if n % 16 or k % 128:
        raise ValueError("n must be a multiple of 16 and k of 128")
    panels = []
    for c0 in range(0, k, 128 * PANEL_BLOCKS):
        cols = qw[:, c0:c0 + 128 * PANEL_BLOCKS]
        ipp = cols.shape[1] // 128
        view = cols.reshape(n // 16, 16, ipp, 2, 4, 16)      # rb, r, j, h, g, e
        panels.append(np.ascontiguousarray(view.transpose(0, 2, 3, 4, 1, 5)).reshape(-1))
    if not panels:
        return np.zeros(0, np.uint8)
    return np.concatenate(panels)
