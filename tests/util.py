"""Small helpers shared by the tests (no attention arithmetic here)."""
import numpy as np


def rel_rms(x, ref):
    """||x - ref||_2 / ||ref||_2 over the whole tensor, in float64 (the
    relative RMS error the pages' tolerance is stated in)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return num
    return num / den
