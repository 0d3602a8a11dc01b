"""Comparison metrics shared by the GPU parity tests (no torch / GPU needed)."""
import numpy as np


def metrics(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    err = np.abs(g - o)
    return {"max_abs": float(err.max()) if err.size else 0.0,
            "mean_rel": float(err.sum() / max(np.abs(o).sum(), 1e-30))}
