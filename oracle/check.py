"""Pass criteria of the parity tests — test infrastructure only.

* Quantized activation and weight bytes and their float32 scales are unique
  under the oracle's readings, so they must match bit for bit.
* The bfloat16 outputs depend on the order and the internal precision of
  the float32 accumulation on the GPU, so they are compared with the
  oracle's float64 value elementwise, with a relative tolerance of 1e-2
  against the oracle's output magnitude.  Reading of "the output
  magnitude": for element (m, n) it is
  ``max(|y64[m, n]|, RMS_FLOOR * rms(y64[m, :]))`` with RMS_FLOOR = 2^-3:
  an element at least an eighth of the token's output-row RMS is held to
  1 % of its own value, a smaller one to 1.25e-3 of the row RMS.  The floor
  comes from the arithmetic of FP8 matrix instructions: the products inside
  one instruction are summed in fixed point about 13 bits below the largest
  product, so an output that cancels to near zero carries an absolute error
  that is a small fraction of the row RMS, which a purely relative test
  cannot absorb.  Measured over every output comparison of the GPU tests,
  the largest such error is 7.8e-4 of the row RMS (random E4M3 codes, whose
  products span 2^36) and 3.7e-4 on the model-shaped workloads, so 1.25e-3
  leaves a margin of 1.6x and 3.4x; a wrong scale, index or dropped K block
  moves elements by far more.  A row whose oracle output is all zero must
  be exactly +-0.  NaN or infinity in the GPU output is always a failure.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, f64_to_bf16_bits

REL_TOL = 1e-2
RMS_FLOOR = 2.0 ** -3


def check_bytes(got: np.ndarray, want: np.ndarray, what: str = "bytes"):
    """Raise AssertionError with the first mismatches unless equal bit for bit."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        raise AssertionError(f"{what}: shape {got.shape} != {want.shape}")
    if got.dtype.itemsize != want.dtype.itemsize:
        raise AssertionError(f"{what}: itemsize differs")
    g = got.view(np.dtype(f"u{got.dtype.itemsize}"))
    w = want.view(np.dtype(f"u{want.dtype.itemsize}"))
    bad = np.argwhere(g != w)
    if bad.size:
        first = [tuple(int(i) for i in b) for b in bad[:8]]
        detail = ", ".join(f"{i}: got {g[i]:#x} want {w[i]:#x}" for i in first)
        raise AssertionError(f"{what}: {len(bad)} mismatches; first {detail}")


#: Every check_close call appends a summary here (what was compared, the
#: largest error over the row RMS, the smallest floor that would still pass
#: and the largest relative error); tests/conftest.py can write the list out
#: so that the measured margins of a run are on record.
REPORT_LOG = []


def close_report(y_bf16_bits: np.ndarray, y64: np.ndarray) -> dict:
    """Elementwise comparison data (no assertion).

    ``floor_needed`` is the smallest RMS floor (in units of the row RMS)
    under which every element would pass: the largest ``err / (REL_TOL *
    rms)`` over the elements whose error exceeds ``REL_TOL * |y64|``."""
    y = bf16_bits_to_f32(y_bf16_bits).astype(np.float64)
    y64 = np.asarray(y64, dtype=np.float64)
    if y.shape != y64.shape:
        raise AssertionError(f"output shape {y.shape} != {y64.shape}")
    rms = np.sqrt(np.mean(y64 * y64, axis=-1, keepdims=True)) if y64.size \
        else np.zeros(y64.shape[:-1] + (1,))
    ref = np.maximum(np.abs(y64), RMS_FLOOR * rms)
    err = np.abs(y - y64)
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(ref > 0, err / np.where(ref > 0, ref, 1.0),
                       np.where(err > 0, np.inf, 0.0))
    finite = np.isfinite(y)
    exact_bf16 = f64_to_bf16_bits(y64) == np.asarray(y_bf16_bits, np.uint16)
    err_rms = np.where(rms > 0, err / np.where(rms > 0, rms, 1.0),
                       np.where(err > 0, np.inf, 0.0)) if rel.size else rel
    beyond = err > REL_TOL * np.abs(y64)
    floor_needed = float(np.max(np.where(beyond, err_rms, 0.0))) / REL_TOL \
        if rel.size else 0.0
    return {
        "max_rel": float(np.max(rel)) if rel.size else 0.0,
        "max_err_over_rms": float(np.max(err_rms)) if rel.size else 0.0,
        "floor_needed": floor_needed,
        "worst_index": tuple(int(i) for i in np.unravel_index(
            np.argmax(rel), rel.shape)) if rel.size else (),
        "n_bad": int(np.sum((rel > REL_TOL) | ~finite)),
        "all_finite": bool(np.all(finite)),
        "frac_bf16_equal": float(np.mean(exact_bf16)) if rel.size else 1.0,
        "rel": rel,
    }


def check_close(y_bf16_bits: np.ndarray, y64: np.ndarray, what="output"):
    """Raise unless every element is within the elementwise tolerance."""
    r = close_report(y_bf16_bits, y64)
    REPORT_LOG.append({"what": what, "max_err_over_rms": r["max_err_over_rms"],
                       "floor_needed": r["floor_needed"], "max_rel": r["max_rel"],
                       "frac_bf16_equal": r["frac_bf16_equal"], "n_bad": r["n_bad"],
                       "elements": int(np.asarray(y64).size)})
    if r["n_bad"]:
        idx = r["worst_index"]
        y = bf16_bits_to_f32(np.asarray(y_bf16_bits, np.uint16))
        raise AssertionError(
            f"{what}: {r['n_bad']} elements out of tolerance; worst at {idx}: "
            f"got {float(y[idx])!r} want {float(np.asarray(y64)[idx])!r} "
            f"rel {r['max_rel']:.3g}; max error / row RMS "
            f"{r['max_err_over_rms']:.3g} (floor {RMS_FLOOR:g} x RMS; this run "
            f"needs {r['floor_needed']:.3g})")
    return r
