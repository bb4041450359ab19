"""The accept rules of the verifier step (oracle; test infrastructure only):
the p/q accept/reject rule with residual resampling, target-sample matching,
and the per-step accounting of the yield-quench policy.

Source: *Optimizing DeepSeek-V4-Flash on a single NVIDIA GB10/GX10 with DSpark
speculative decoding*, post 1, the paragraph under the analyzer output: the
drafts are sampled from q, the target model defines p, a draft x is accepted
with probability min(1, p(x)/q(x)), and a rejected draft is replaced by a
sample of the positive residual distribution (normalised max(0, p - q)).  The
verifier pushes K+1 rows -- the committed position plus the K drafts -- through
the target (page 2 of the same thread, the author's verifier post; *ds4-on-spark*
README, "The break-even law": one committed row plus four draft rows), so when
every draft passes, row K yields one more token (the bonus token).

The steps, per sequence, with uniforms u_0 .. u_K given as inputs:

  for i = 0 .. K-1, d = draft i:
      accept iff u_i * q_i(d) < p_i(d)                (exact comparison)
      on reject: r = max(0, p_i - q_i); emit the first x (vocabulary order) whose
                 running sum C(x) = sum_{y <= x} r(y) exceeds u_K * Z, Z = C(V-1);
                 if Z == 0 sample p_i the same way instead; stop
  all K accepted: emit the same inverse-CDF sample of p_K (the bonus token)

Readings where the pages are silent (listed in the design notes): the uniform
budget (K accept uniforms plus one sampling uniform), inverse-CDF order
(vocabulary index, strict ">"), equality rejects, the Z == 0 fallback, and the
bonus row.

``p`` and ``q`` come either from logits (softmax at temperature T, fp64) or are
given as probabilities.  T = 0 is greedy decoding (the same thread, page 1, post
12: greedy outputs unchanged; *1x Spark tuned DSpark for DeepSeek-V4-Flash*,
Q&A, the FP8 KV answer: the speculative self-check exact at temperature 0): the row is the one-hot distribution at its largest logit, the limit of the
softmax as T falls to 0, with ties going to the lowest index (our reading; the
limit itself would split the mass over tied maxima).  ``accept_sequence`` also runs on ``fractions.Fraction``
inputs, where every step is exact; the parity pins enumerate it that way.
"""
from __future__ import annotations

from fractions import Fraction
from itertools import accumulate
from typing import List, Sequence, Tuple

import numpy as np

LOGITS, PROBS = 0, 1


def softmax_t(z, temperature: float) -> np.ndarray:
    """p = exp(z/T - max) / sum, fp64, for one row of fp32 logits."""
    a = np.asarray(z, np.float32).astype(np.float64) / np.float64(np.float32(temperature))
    e = np.exp(a - a.max())
    return e / e.sum()


def greedy_onehot(z) -> np.ndarray:
    """The T = 0 distribution of one row of fp32 logits: 1 at the first index
    holding the row's maximum, 0 elsewhere (fp64)."""
    a = np.asarray(z, np.float32)
    p = np.zeros(a.shape[0], np.float64)
    p[int(np.argmax(a))] = 1.0   # numpy's argmax returns the first maximum
    return p


def distribution(row, kind: int, temperature: float) -> np.ndarray:
    """p (or q) of one row: softmax at T, the T = 0 one-hot, or the given
    probabilities (fp64)."""
    if kind == PROBS:
        return np.asarray(row, np.float32).astype(np.float64)
    if np.float32(temperature) == 0:
        return greedy_onehot(row)
    return softmax_t(row, temperature)


def first_exceeding(weights, u):
    """Index of the first x with sum_{y<=x} w(y) > u * Z, Z = total mass.

    Runs on an fp64 numpy row (running sum in index order, fp64) or on a list
    of Fractions (exact).  Returns None when Z <= 0.
    """
    if isinstance(weights, np.ndarray):
        c = np.cumsum(weights, dtype=np.float64)
        z = c[-1]
        if not z > 0.0:
            return None
        t = np.float64(u) * z
        return int(np.argmax(c > t))
    c = list(accumulate(weights))
    z = c[-1]
    if not z > 0:
        return None
    t = Fraction(u) * z
    for x, cx in enumerate(c):
        if cx > t:
            return x
    return None   # unreachable for u < 1


def _lt_exact(a, b, c) -> bool:
    """a * b < c, evaluated exactly."""
    return Fraction(a) * Fraction(b) < Fraction(c)


def _residual(p, q):
    if isinstance(p, np.ndarray):
        return np.maximum(p - q, 0.0)
    return [max(Fraction(0), pi - qi) for pi, qi in zip(p, q)]


def accept_sequence(p_rows: Sequence, q_rows: Sequence, drafts: Sequence[int],
                    u: Sequence) -> Tuple[int, List[int]]:
    """One sequence: p_rows K+1 distributions, q_rows K, drafts K, u K+1.

    Returns (n_accepted, emitted tokens: n_accepted drafts then one more)."""
    K = len(drafts)
    out: List[int] = []
    for i in range(K):
        d = int(drafts[i])
        if _lt_exact(u[i], q_rows[i][d], p_rows[i][d]):
            out.append(d)
            continue
        tok = first_exceeding(_residual(p_rows[i], q_rows[i]), u[K])
        if tok is None:
            tok = first_exceeding(p_rows[i], u[K])
        out.append(tok)
        return i, out
    out.append(first_exceeding(p_rows[K], u[K]))
    return K, out


def _row_valid(v: np.ndarray, kind: int) -> bool:
    if not np.all(np.isfinite(v)):
        return False
    if kind == PROBS:
        return bool(np.all(v >= 0)) and float(v.astype(np.float64).sum()) > 0.0
    return True


def spec_accept(S: int, K: int, V: int, target, target_kind: int, t_p: float,
                draft, draft_kind: int, t_q: float, drafts, uniforms):
    """Batched form with the library's argument order.

    target [S*(K+1), V] fp32 (row s*(K+1)+i), draft [S*K, V] fp32, drafts
    [S, K] int32, uniforms [S, K+1] fp32.  Returns (out_tokens int32 [S, K+1]
    padded with -1, n_accepted int32 [S]); a sequence whose inputs are invalid
    (a token outside [0, V), a uniform outside [0, 1), a non-finite value, or a
    negative / all-zero probability row) gets -1 everywhere.
    """
    target = np.asarray(target, np.float32).reshape(S, K + 1, V)
    draft = np.asarray(draft, np.float32).reshape(S, K, V) if K else np.zeros((S, 0, V), np.float32)
    drafts = np.asarray(drafts, np.int64).reshape(S, K)
    uniforms = np.asarray(uniforms, np.float32).reshape(S, K + 1)
    toks = np.full((S, K + 1), -1, np.int32)
    nacc = np.full(S, -1, np.int32)
    for s in range(S):
        ok = all(_row_valid(target[s, i], target_kind) for i in range(K + 1))
        ok = ok and all(_row_valid(draft[s, i], draft_kind) for i in range(K))
        ok = ok and bool(np.all((drafts[s] >= 0) & (drafts[s] < V)))
        ok = ok and bool(np.all((uniforms[s] >= 0) & (uniforms[s] < 1)))
        if not ok:
            continue

        p_rows = [distribution(target[s, i], target_kind, t_p) for i in range(K + 1)]
        q_rows = [distribution(draft[s, i], draft_kind, t_q) for i in range(K)]
        n, out = accept_sequence(p_rows, q_rows, drafts[s].tolist(),
                                 [float(x) for x in uniforms[s]])
        nacc[s] = n
        toks[s, :len(out)] = out
    return toks, nacc


def target_sample_sequence(p_rows: Sequence, drafts: Sequence[int],
                           u: Sequence) -> Tuple[int, List[int]]:
    """Target-sample matching for one sequence: p_rows K+1 distributions,
    drafts K, u K+1.

    Source: *1x Spark tuned DSpark for DeepSeek-V4-Flash*, the paragraph on
    losslessness under "The break-even law, and why speculation can't hurt you
    here": the verify rows are the only source of tokens; the accept loop
    draws the target's own token from each verify row with the request's
    sampler and random stream.  Steps: for i = 0 .. K, t_i = the inverse-CDF
    sample of p_i at u_i (the first x whose running sum exceeds u_i times the
    row total, as for the p/q rule's sample); while i < K and t_i equals
    draft i the draft stands and the walk moves on to row i+1; the first t_i
    that differs (or t_K) is emitted and ends the step.  The draft rows q are
    not used.  Returns (n_accepted, emitted tokens: n_accepted drafts, then
    t_n)."""
    K = len(drafts)
    out: List[int] = []
    for i in range(K + 1):
        t = first_exceeding(p_rows[i], u[i])
        out.append(t)
        if i == K or t != int(drafts[i]):
            return i, out
    raise AssertionError("unreachable")


def spec_accept_target_sample(S: int, K: int, V: int, target, target_kind: int, t_p: float,
                              drafts, uniforms):
    """Batched target-sample matching with the library's argument order:
    target [S*(K+1), V] fp32 (row s*(K+1)+i), drafts [S, K] int32, uniforms
    [S, K+1] fp32 (u[s][i] samples row i).  Returns (out_tokens int32
    [S, K+1] padded with -1, n_accepted int32 [S]); invalid inputs (a token
    outside [0, V), a uniform outside [0, 1), a non-finite value, a negative
    or all-zero probability row) give -1 everywhere for that sequence."""
    target = np.asarray(target, np.float32).reshape(S, K + 1, V)
    drafts = np.asarray(drafts, np.int64).reshape(S, K)
    uniforms = np.asarray(uniforms, np.float32).reshape(S, K + 1)
    toks = np.full((S, K + 1), -1, np.int32)
    nacc = np.full(S, -1, np.int32)
    for s in range(S):
        ok = all(_row_valid(target[s, i], target_kind) for i in range(K + 1))
        ok = ok and bool(np.all((drafts[s] >= 0) & (drafts[s] < V)))
        ok = ok and bool(np.all((uniforms[s] >= 0) & (uniforms[s] < 1)))
        if not ok:
            continue
        p_rows = [distribution(target[s, i], target_kind, t_p) for i in range(K + 1)]
        n, out = target_sample_sequence(p_rows, drafts[s].tolist(), [float(x) for x in uniforms[s]])
        nacc[s] = n
        toks[s, :len(out)] = out
    return toks, nacc


def yield_quench(n_accepted_steps: Sequence[int], guard, threshold):
    """The per-request accounting of the yield-quench policy over a run of
    verify steps.

    Source: *ds4-on-spark* README, "The break-even law" (a verify step costs
    about as much as `guard` plain decode steps, so it pays only when it
    commits more tokens than that; the controller sums the regret
    guard - tokens-per-step over the verify steps and turns speculation off
    for the rest of the request once the sum exceeds a few plain-step
    times), and *1x Spark tuned DSpark for DeepSeek-V4-Flash*, "The break-even
    law, and why speculation can't hurt you here" (the realised regret
    guard - tokens committed, accumulated per verify step; the quench is
    terminal).  Steps, for each step's accepted-draft count n (-1: the
    sequence's inputs were invalid, nothing committed, not counted): tokens
    committed t = n + 1; steps += 1; tokens += t; regret += guard - t; once
    regret > threshold the request is quenched at that step and later steps
    are not counted.  Readings (listed in the design notes): the sum is not
    clamped at zero (a request that runs ahead banks credit), "exceeds" is
    strict, and the regret is a plain running sum in the arithmetic of its
    inputs (fp64 floats, or exact Fractions).

    Returns (steps, tokens, regret, quench_step or None)."""
    steps = tokens = 0
    regret = guard - guard   # zero in the inputs' arithmetic
    for n in n_accepted_steps:
        if n < 0:
            continue
        t = int(n) + 1
        steps += 1
        tokens += t
        regret = regret + (guard - t)
        if regret > threshold:
            return steps, tokens, regret, steps
    return steps, tokens, regret, None
