"""Error metrics shared by the GPU parity tests.

Relative error of a result x against the oracle r is measured per
(instance, head) slab as max|x - r| / max|r| over that slab (tokens x dv for
outputs, dv x dk for a state), and the worst slab is reported.
"""
import numpy as np

OUT_TOL = 2e-3     # outputs, bf16 or fp32 inputs with fp32 state
STATE_TOL = 1e-3   # committed / final state


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_err_outputs(o, ref):
    """o, ref: [B][T][H][dv] -> worst slab error over (instance, head)."""
    o, ref = _np(o), _np(ref)
    diff = np.abs(o - ref).max(axis=(1, 3))
    scale = np.abs(ref).max(axis=(1, 3))
    return float((diff / np.maximum(scale, 1e-300)).max())


def rel_err_state(S, ref):
    """S, ref: [B][H][dv][dk] -> worst slab error over (instance, head)."""
    S, ref = _np(S), _np(ref)
    diff = np.abs(S - ref).max(axis=(2, 3))
    scale = np.abs(ref).max(axis=(2, 3))
    return float((diff / np.maximum(scale, 1e-300)).max())
