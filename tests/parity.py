"""Shared helpers for the GPU parity tests: tolerances and comparisons.

Tolerances on O: bf16 inputs max-abs 2e-2 and mean-abs 2e-3; fp32 inputs
1e-5.  On LSE: 1e-3 (bf16) and 1e-5 (fp32).  Where the oracle gives -inf
(no visible key) the GPU must give -inf too; NaN is never accepted.
"""
import numpy as np
import torch

TOL = {
    "bf16": {"max_abs": 2e-2, "mean_abs": 2e-3, "lse": 1e-3},
    "f32": {"max_abs": 1e-5, "mean_abs": 1e-5, "lse": 1e-5},
}


def to_f64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def check(got_o, want_o, got_lse, want_lse, dtype, what=""):
    """Compare O and LSE against the oracle; returns (max_abs, mean_abs, lse_err)."""
    tol = TOL[dtype]
    go, wo = to_f64(got_o), to_f64(want_o)
    assert go.shape == wo.shape, (what, go.shape, wo.shape)
    assert np.all(np.isfinite(go)), f"{what}: non-finite output"
    err = np.abs(go - wo)
    max_abs = float(err.max()) if err.size else 0.0
    mean_abs = float(err.mean()) if err.size else 0.0
    assert max_abs <= tol["max_abs"], f"{what}: O max-abs {max_abs:.3e} > {tol['max_abs']}"
    assert mean_abs <= tol["mean_abs"], f"{what}: O mean-abs {mean_abs:.3e} > {tol['mean_abs']}"
    lse_err = 0.0
    if got_lse is not None:
        gl, wl = to_f64(got_lse), to_f64(want_lse)
        assert gl.shape == wl.shape
        assert not np.any(np.isnan(gl)), f"{what}: NaN in LSE"
        inf = np.isinf(wl)
        assert np.array_equal(np.isinf(gl), inf), f"{what}: -inf LSE pattern differs"
        if (~inf).any():
            lse_err = float(np.abs(gl[~inf] - wl[~inf]).max())
        assert lse_err <= tol["lse"], f"{what}: LSE max-abs {lse_err:.3e} > {tol['lse']}"
    return max_abs, mean_abs, lse_err
