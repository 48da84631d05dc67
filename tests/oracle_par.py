"""Row-parallel calls of the oracle for the full-size parity tests (test
orchestration only: each row is quantized on its own by definition, so the
rows are split over threads and the oracle's results concatenated; no
arithmetic here)."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

POOL = 16


def quant_rows_par(bits: np.ndarray, weight: bool = False):
    """oracle.quant_act_ref (or quant_weight_ref) of every row of `bits`."""
    fn = oracle.quant_weight_ref if weight else oracle.quant_act_ref
    if bits.shape[0] < 2 * POOL:
        return fn(bits)
    chunks = np.array_split(np.arange(bits.shape[0]), POOL)
    with ThreadPoolExecutor(POOL) as ex:
        parts = list(ex.map(lambda r: fn(bits[r[0]:r[-1] + 1]), chunks))
    return (np.concatenate([p[0] for p in parts]),
            np.concatenate([p[1] for p in parts]))
