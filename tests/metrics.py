"""Error metrics shared by the tests (no method arithmetic here)."""
import numpy as np


def normwise_rel_err(Y, Yref, axes=(-2, -1)):
    """max over slices of max|Y - Yref| / max|Yref|, a slice being the trailing `axes`.

    Outputs are convex combinations of zero-mean values, so elements near zero
    make an element-wise ratio meaningless; the error is measured against the
    largest reference magnitude of each (batch, head) slice instead.
    """
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    diff = np.max(np.abs(Y - Yref), axis=axes)
    scale = np.max(np.abs(Yref), axis=axes)
    scale = np.where(scale > 0, scale, 1.0)
    return float(np.max(diff / scale))


def rel_err(Y, Yref):
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    s = np.max(np.abs(Yref))
    return float(np.max(np.abs(Y - Yref)) / (s if s > 0 else 1.0))
