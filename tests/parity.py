"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
import numpy as np


def to_np(t):
    if t is None:
        return None
    if hasattr(t, "detach"):
        return t.detach().double().cpu().numpy()
    return np.asarray(t, dtype=np.float64)


def scaled_error(got, want):
    """max|got - want| / max|want| (the scaled error of the OneModel checks)."""
    got, want = to_np(got), to_np(want)
    assert got.shape == want.shape, (got.shape, want.shape)
    den = np.max(np.abs(want)) if want.size else 0.0
    num = np.max(np.abs(got - want)) if want.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)


def assert_close(name, got, want, tol):
    err = scaled_error(got, want)
    print(f"  {name}: scaled error {err:.3e} (tol {tol:g})", flush=True)
    assert err <= tol, f"{name}: scaled error {err:.3e} > {tol:g}"
