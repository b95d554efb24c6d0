"""Error metrics shared by the GPU parity tests (plain NumPy, no attention arithmetic)."""

import numpy as np


def to64(t):
    return t.detach().to("cpu").to(__import__("torch").float64).numpy()


def errs(got, want, rows=None):
    """(max-abs, mean-abs) of got - want, optionally restricted to a boolean row mask."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    if rows is not None:
        got, want = got[rows], want[rows]
    d = np.abs(got - want)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def bf16_floor(want):
    """max |bf16(x) - x| over the reference: the error output rounding alone costs."""
    import torch

    x = torch.from_numpy(np.ascontiguousarray(want))
    return float((x.to(torch.bfloat16).to(torch.float64) - x).abs().max())
