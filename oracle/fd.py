"""Central finite differences in float64.  TEST INFRASTRUCTURE ONLY."""
import numpy as np


def grad(f, x, idx=None, rel_step=1e-6):
    """Central-difference gradient of the scalar function f at x (f takes an
    array shaped like x).  idx: iterable of flat indices to probe (all if
    None).  The step at entry i is rel_step * max(1, |x_i|)."""
    x = np.array(x, np.float64, copy=True)
    flat = x.reshape(-1)
    out = np.zeros(flat.size)
    todo = range(flat.size) if idx is None else idx
    for i in todo:
        h = rel_step * max(1.0, abs(flat[i]))
        keep = flat[i]
        flat[i] = keep + h
        fp = f(x)
        flat[i] = keep - h
        fm = f(x)
        flat[i] = keep
        out[i] = (fp - fm) / (2.0 * h)
    return out.reshape(x.shape)


def rel_err(a, b):
    """||a - b||_inf / ||b||_inf (the per-tensor error measure)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))
