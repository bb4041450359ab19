"""Parity helpers shared by the GPU tests (comparison metric and flags).

Floating-point bar: max relative error 2e-3 against the oracle, read per output
row as err_i = |y_i - yhat_i| / max(|yhat_i|, 1e-3 * max_j |yhat_j|), so that
outputs near zero are measured against the row's scale instead of failing on
meaningless relative errors.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 2e-3
FLOOR = 1e-3
FLAG_BAND = 1e-6

# (what, worst row-relative error, tolerance) of every comparison made in this
# process; printed at the end of the run (tests/conftest.py)
MARGINS = []


def rel_err_rows(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if want.ndim == 1:
        want = want[None]
        got = got[None]
    scale = np.max(np.abs(want), axis=1, keepdims=True)
    den = np.maximum(np.abs(want), FLOOR * scale)
    den = np.where(den > 0, den, 1.0)
    return np.abs(got - want) / den


def assert_close(got, want, tol: float = REL_TOL, what: str = ""):
    e = rel_err_rows(got, want)
    worst = float(e.max()) if e.size else 0.0
    MARGINS.append((what, worst, tol))
    assert np.all(np.isfinite(np.asarray(got, np.float64))), f"{what}: non-finite output"
    assert worst <= tol, f"{what}: max row-relative error {worst:.3e} > {tol:.1e}"
    return worst


def accept_flags(p_rows, q_rows, drafts, u, n_oracle):
    """Decisions of the oracle run that sit within the flag band: an accept
    test with |u - p/q| < 1e-6 among the tests the oracle made."""
    flagged = False
    for i in range(min(n_oracle + 1, len(drafts))):
        d = int(drafts[i])
        q = float(q_rows[i][d])
        p = float(p_rows[i][d])
        if q > 0 and abs(float(u[i]) - p / q) < FLAG_BAND:
            flagged = True
    return flagged


def sample_flag(weights: np.ndarray, u: float) -> bool:
    """True if u * Z lies within 1e-6 * Z of a CDF boundary."""
    c = np.cumsum(np.asarray(weights, np.float64))
    z = c[-1]
    if not z > 0:
        return False
    t = float(u) * z
    return bool(np.any(np.abs(c - t) < FLAG_BAND * z))
