"""Comparison metric used by the parity tests (oracle; test infrastructure only)."""
import numpy as np


def normwise_rel_err(y, ref):
    """max over rows m of  max_o |y[m,o] - ref[m,o]| / max_o |ref[m,o]|.

    An elementwise relative gate fails near-zero outputs even for exact
    float32 kernels, so the 1e-3 tolerance is applied row-normwise.  Returns
    (err, min row scale) so that callers can require a non-trivial magnitude.
    """
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    r = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    scale = np.max(np.abs(r), axis=1)
    diff = np.max(np.abs(y - r), axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(scale > 0, diff / scale, np.where(diff > 0, np.inf, 0.0))
    return float(np.max(rel)), float(np.min(scale))
