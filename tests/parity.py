"""Parity helpers shared by the GPU tests.

Tolerances (max abs error over every compared element, in units of the
oracle's RMS over the same tensor):
  fp32 q/k/v:            1e-4
  bf16 q/k/v, fp32 state: 2e-2
States are compared the same way against the RMS of the oracle's state.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref):
    """max |got - ref| / RMS(ref) over the elements where ref is defined (not NaN)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    if not m.any():
        raise ValueError("nothing to compare")
    r = ref[m]
    rms = float(np.sqrt(np.mean(r * r)))
    if rms == 0.0:
        return float(np.max(np.abs(got[m] - r)))
    return float(np.max(np.abs(got[m] - r)) / rms)


def assert_parity(got, ref, tol, what):
    err = rel_err(got, ref)
    print(f"[parity] {what}: max|err|/RMS = {err:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64)[~np.isnan(ref)])), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max|err|/RMS = {err:.3e} > {tol:.0e}"
    return err
