"""Comparison of stored floating-point results (shared by the GPU harness and
its CPU test)."""
import numpy as np


def same_floats32(got: np.ndarray, want: np.ndarray) -> bool:
    """Binary32 arrays equal bit for bit, except that an element that is NaN
    on both sides matches whatever its NaN bits: IEEE 754 leaves the sign and
    payload of a NaN result unspecified when an add makes a NaN or meets one,
    and the oracle's CPU add and the GPU's choose differently.  Where either
    side is NaN the other must be NaN too."""
    gn, wn = np.isnan(got), np.isnan(want)
    if not np.array_equal(gn, wn):
        return False
    keep = ~gn
    return np.array_equal(got[keep].view(np.uint32), want[keep].view(np.uint32))
