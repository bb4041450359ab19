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


def check_target_sample(S, K, V, target, tk, tp, drafts, u, toks, nacc):
    """GPU target-sample matching against the oracle on the same inputs:
    invalid sequences all -1; otherwise n_accepted and tokens equal, except
    from the first row the oracle sampled whose u * Z lies within 1e-6 * Z of
    a CDF boundary (before that row the outputs must still agree).  Returns
    (oracle n_accepted, number of flagged sequences)."""
    import oracle
    wt, wn = oracle.spec_accept_target_sample(S, K, V, target, tk, tp, drafts, u)
    tg = np.asarray(target, np.float32).reshape(S, K + 1, V)
    flagged = 0
    for s in range(S):
        if wn[s] < 0:
            assert nacc[s] == -1 and np.all(toks[s] == -1), f"sequence {s}: {nacc[s]} {toks[s]}"
            continue
        n = int(wn[s])
        fl = [sample_flag(oracle.distribution(tg[s, i], tk, tp), u[s, i]) for i in range(n + 1)]
        if any(fl):
            j = fl.index(True)
            assert nacc[s] >= j and np.array_equal(toks[s, :j], wt[s, :j]), f"sequence {s}"
            flagged += 1
            continue
        assert nacc[s] == n and np.array_equal(toks[s], wt[s]), (
            f"sequence {s}: n {nacc[s]} tokens {toks[s]} vs oracle {n} {wt[s]}")
    return wn, flagged


def matching_drafts(S, K, V, target, tk, tp, u, p_match, rng):
    """Drafts that equal the target's own sample of their row (the oracle's,
    at the same uniform) with probability p_match, else uniform tokens: inputs
    for target-sample matching whose accepted prefixes take every length."""
    import oracle
    tg = np.asarray(target, np.float32).reshape(S, K + 1, V)
    d = rng.integers(0, V, size=(S, K)).astype(np.int32)
    for s in range(S):
        for i in range(K):
            if rng.random() < p_match:
                d[s, i] = oracle.first_exceeding(oracle.distribution(tg[s, i], tk, tp), float(u[s, i]))
    return d
