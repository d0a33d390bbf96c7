"""Error metrics used by the parity tests (test-side only)."""
import numpy as np


def r3(y, y_ref, scale_ref):
    """max |y - y*| / max(|y*|, S*), S* = sum p|v| / sum p: relative error against the magnitude
    the weighted mean is formed from (plain |y - y*| / |y*| is ill-posed where y* crosses zero)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    denom = np.maximum(np.abs(y_ref), np.asarray(scale_ref, dtype=np.float64))
    denom = np.where(denom > 0, denom, 1.0)
    return float(np.max(np.abs(y - y_ref) / denom)) if y.size else 0.0


def r2(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    m = float(np.max(np.abs(y_ref))) if y.size else 0.0
    return float(np.max(np.abs(y - y_ref))) / m if m > 0 else 0.0
