"""Pins of the oracle's accept/reject rule (CPU only).

The key pin is exact enumeration: on tiny vocabularies the emitted-token
distribution of the oracle, driven cell by cell through every region of its
uniforms, must equal the target distribution exactly, whatever the draft
distribution q -- the losslessness the pages claim for the p/q rule.
"""
import itertools
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.accept import LOGITS, PROBS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F = Fraction


def test_golden_cases():
    for c in json.load(open(os.path.join(GOLDEN, "accept_v4.json")))["cases"]:
        p = [[F(v) for v in row] for row in c["p"]]
        q = [[F(v) for v in row] for row in c["q"]]
        n, toks = oracle.accept_sequence(p, q, c["drafts"], [F(v) for v in c["u"]])
        assert (n, toks) == (c["n_accepted"], c["tokens"]), c["name"]
        if c.get("fp64_boundary"):
            continue
        # the fp64 path agrees away from decision boundaries
        pn = [np.array([float(v) for v in row]) for row in p]
        qn = [np.array([float(v) for v in row]) for row in q]
        n2, t2 = oracle.accept_sequence(pn, qn, c["drafts"], [float(F(v)) for v in c["u"]])
        assert (n2, t2) == (n, toks), c["name"]


def test_softmax_closed_forms():
    V = 17
    assert np.allclose(oracle.softmax_t(np.full(V, 3.25, np.float32), 0.8), 1.0 / V, rtol=1e-15)
    z = np.random.default_rng(0).normal(size=50).astype(np.float32)
    p = oracle.softmax_t(z, 1.3)
    assert abs(p.sum() - 1.0) < 1e-15
    p2 = oracle.softmax_t((z + np.float32(4.0)).astype(np.float32), 1.3)
    assert np.allclose(p, p2, rtol=1e-6)          # shift invariance (z+4 rounds in fp32)
    a, b, t = np.float32(1.5), np.float32(-0.25), 0.7
    pr = oracle.softmax_t(np.array([a, b]), t)
    sig = 1.0 / (1.0 + math.exp(-(float(a) - float(b)) / float(np.float32(t))))
    assert abs(pr[0] - sig) < 1e-15 and abs(pr[1] - (1 - sig)) < 1e-15


def _rand_dist(rng, V, zero_prob):
    while True:
        w = [0 if rng.random() < zero_prob else rng.randint(1, 9) for _ in range(V)]
        if sum(w):
            s = sum(w)
            return [F(x, s) for x in w]


def _cells_inverse_cdf(w):
    """[(x, lo, hi)]: u in [lo, hi) picks x by the first-exceeding rule."""
    z = sum(w)
    out, c = [], F(0)
    for x, wx in enumerate(w):
        if wx > 0:
            out.append((x, c / z, (c + wx) / z))
        c += wx
    return out


def _enumerate(V, K, p_tab, q_tab):
    """Emitted-prefix distribution of the oracle, by driving it with the
    midpoint of every decision cell; also asserts the oracle's decisions match
    the cells (and equality at a boundary rejects)."""
    dist = {}
    for drafts in itertools.product(range(V), repeat=K):
        wq = F(1)
        for i in range(K):
            wq *= q_tab[drafts[:i]][drafts[i]]
        if wq == 0:
            continue
        p_rows = [p_tab[drafts[:i]] for i in range(K + 1)]
        q_rows = [q_tab[drafts[:i]] for i in range(K)]
        for n in range(K + 1):          # accept n drafts, then reject (n < K) or bonus (n == K)
            us = []
            prob = wq
            ok = True
            for i in range(n):
                a = min(F(1), p_rows[i][drafts[i]] / q_rows[i][drafts[i]])
                if a == 0:
                    ok = False
                    break
                us.append(a / 2)
                prob *= a
            if not ok:
                continue
            if n < K:
                a = min(F(1), p_rows[n][drafts[n]] / q_rows[n][drafts[n]])
                if a == 1:
                    continue
                us.append((a + 1) / 2)
                prob *= 1 - a
                res = [max(F(0), pi - qi) for pi, qi in zip(p_rows[n], q_rows[n])]
                cells = _cells_inverse_cdf(res)
            else:
                cells = _cells_inverse_cdf(p_rows[K])
            us += [F(0)] * (K - len(us))
            for x, lo, hi in cells:
                u = us + [(lo + hi) / 2]
                got_n, toks = oracle.accept_sequence(p_rows, q_rows, list(drafts), u)
                want = list(drafts[:n]) + [x]
                assert (got_n, toks) == (n, want)
                key = tuple(want)
                dist[key] = dist.get(key, F(0)) + prob * (hi - lo)
                # the cell's lower edge belongs to x as well (strict ">" rule)
                got_n2, toks2 = oracle.accept_sequence(p_rows, q_rows, list(drafts), us + [lo])
                assert toks2[-1] == x
            if n < K:
                # a uniform exactly at p/q rejects
                a = min(F(1), p_rows[n][drafts[n]] / q_rows[n][drafts[n]])
                u_edge = us[:n] + [a] + [F(0)] * (K - n - 1) + [F(1, 2)]
                assert oracle.accept_sequence(p_rows, q_rows, list(drafts), u_edge)[0] == n
    return dist


@pytest.mark.parametrize("V,K", [(2, 1), (2, 3), (3, 1), (3, 2), (4, 1), (4, 2), (4, 3)])
def test_exact_enumeration_lossless(V, K):
    rng = random.Random(1000 * V + K)
    for trial in range(3 if V * K > 8 else 6):
        prefixes = [pre for L in range(K + 1) for pre in itertools.product(range(V), repeat=L)]
        p_tab = {pre: _rand_dist(rng, V, 0.25) for pre in prefixes}
        q_tab = {pre: _rand_dist(rng, V, 0.25) for pre in prefixes}
        dist = _enumerate(V, K, p_tab, q_tab)
        # emitted mass sums to one
        assert sum(dist.values()) == 1
        # complete every emitted prefix with target sampling to K+1 tokens
        full = {}
        for pre, m in dist.items():
            for tail in itertools.product(range(V), repeat=K + 1 - len(pre)):
                seq = pre + tail
                w = m
                for j in range(len(pre), K + 1):
                    w *= p_tab[seq[:j]][seq[j]]
                if w:
                    full[seq] = full.get(seq, F(0)) + w
        for seq in itertools.product(range(V), repeat=K + 1):
            target = F(1)
            for j in range(K + 1):
                target *= p_tab[seq[:j]][seq[j]]
            assert full.get(seq, F(0)) == target, (seq, full.get(seq), target)


def test_acceptance_rate_is_one_minus_tv():
    """P(accept first draft) = sum_x min(p(x), q(x))."""
    rng = random.Random(7)
    for _ in range(20):
        V = 5
        p, q = _rand_dist(rng, V, 0.2), _rand_dist(rng, V, 0.2)
        acc = F(0)
        for d in range(V):
            if q[d] == 0:
                continue
            a = min(F(1), p[d] / q[d])
            # check the oracle accepts below a and rejects at a
            if a > 0:
                assert oracle.accept_sequence([p, p], [q], [d], [a / 3, F(0)])[0] == 1
            if a < 1:
                assert oracle.accept_sequence([p, p], [q], [d], [a, F(0)])[0] == 0
            acc += q[d] * a
        assert acc == sum(min(a, b) for a, b in zip(p, q))


def test_special_cases():
    p = [F(1, 10), F(2, 10), F(3, 10), F(4, 10)]
    # q = p: every draft accepted, bonus from p_K
    for d in range(4):
        for u in (F(0), F(1, 2), F(99, 100)):
            n, toks = oracle.accept_sequence([p, p], [p], [d], [u, F(1, 2)])
            assert n == 1 and toks[0] == d
    # q one-hot on d: accepted iff u < p(d); residual is p without d, renormalised
    d = 2
    q = [F(0), F(0), F(1), F(0)]
    assert oracle.accept_sequence([p, p], [q], [d], [F(29, 100), F(0)])[0] == 1
    assert oracle.accept_sequence([p, p], [q], [d], [F(3, 10), F(0)])[0] == 0
    res_cells = _cells_inverse_cdf([F(1, 10), F(2, 10), F(0), F(4, 10)])
    for x, lo, hi in res_cells:
        assert oracle.accept_sequence([p, p], [q], [d], [F(1, 2), (lo + hi) / 2])[1] == [x]
    # disjoint supports: always rejected at step 0, residual = p_0
    p0 = [F(1, 2), F(1, 2), F(0), F(0)]
    q0 = [F(0), F(0), F(1, 2), F(1, 2)]
    for u in (F(0), F(1, 2)):
        n, toks = oracle.accept_sequence([p0, p, p], [q0, q0], [2, 3], [u, u, F(3, 4)])
        assert n == 0 and toks == [1]


def test_batched_form_and_invalid_inputs():
    rng = np.random.default_rng(4)
    S, K, V = 4, 3, 9
    tl = rng.normal(size=(S * (K + 1), V)).astype(np.float32) * 2
    dl = rng.normal(size=(S * K, V)).astype(np.float32)
    drafts = rng.integers(0, V, size=(S, K)).astype(np.int32)
    u = rng.random(size=(S, K + 1)).astype(np.float32)
    toks, nacc = oracle.spec_accept(S, K, V, tl, LOGITS, 1.0, dl, LOGITS, 1.0, drafts, u)
    for s in range(S):
        p_rows = [oracle.softmax_t(tl[s * (K + 1) + i], 1.0) for i in range(K + 1)]
        q_rows = [oracle.softmax_t(dl[s * K + i], 1.0) for i in range(K)]
        n, out = oracle.accept_sequence(p_rows, q_rows, drafts[s].tolist(), [float(x) for x in u[s]])
        assert nacc[s] == n and toks[s, :n + 1].tolist() == out and np.all(toks[s, n + 1:] == -1)
    bad = [drafts.copy(), u.copy(), tl.copy()]
    bad[0][1, 0] = V
    bad[1][2, 3] = 1.0
    bad[2][3 * (K + 1) + 2, 5] = np.nan
    t1, n1 = oracle.spec_accept(S, K, V, tl, LOGITS, 1.0, dl, LOGITS, 1.0, bad[0], u)
    t2, n2 = oracle.spec_accept(S, K, V, tl, LOGITS, 1.0, dl, LOGITS, 1.0, drafts, bad[1])
    t3, n3 = oracle.spec_accept(S, K, V, bad[2], LOGITS, 1.0, dl, LOGITS, 1.0, drafts, u)
    for (t, n, s_bad) in ((t1, n1, 1), (t2, n2, 2), (t3, n3, 3)):
        assert n[s_bad] == -1 and np.all(t[s_bad] == -1)
        keep = [s for s in range(S) if s != s_bad]
        assert np.array_equal(n[keep], nacc[keep]) and np.array_equal(t[keep], toks[keep])
    # probabilities mode: negative entries are invalid
    pr = np.abs(rng.normal(size=(S * (K + 1), V))).astype(np.float32)
    qr = np.abs(rng.normal(size=(S * K, V))).astype(np.float32)
    pr[0, 0] = -1e-3
    t4, n4 = oracle.spec_accept(S, K, V, pr, PROBS, 1.0, qr, PROBS, 1.0, drafts, u)
    assert n4[0] == -1 and np.all(n4[1:] >= 0)


def test_probs_mode_unnormalised_rows():
    """Given probability rows are used as they are: the bonus inverse CDF
    divides by the row's own total."""
    p = [np.array([0.2, 0.2, 0.4, 0.0]), np.array([1.0, 1.0, 2.0, 4.0])]   # second sums to 8
    q = [np.array([0.25, 0.25, 0.25, 0.25])]
    n, toks = oracle.accept_sequence(p, q, [0], [0.5, 0.3])   # 0.125 < 0.2 accept
    # sums 1,2,4,8; target 0.3*8 = 2.4 -> first > 2.4 is x=2
    assert (n, toks) == (1, [0, 2])


def _first_max(row):
    vals = [float(v) for v in row]
    return vals.index(max(vals))   # list.index: the first occurrence


def _prefix_match(tl, drafts, S, K):
    """Greedy decoding written out without the accept rule: drafts are kept
    while each equals its target row's largest logit (the first one on ties);
    the first disagreeing row, or row K, then gives its own largest logit."""
    toks = np.full((S, K + 1), -1, np.int32)
    nacc = np.zeros(S, np.int32)
    for s in range(S):
        best = [_first_max(tl[s * (K + 1) + i]) for i in range(K + 1)]
        n = 0
        while n < K and int(drafts[s][n]) == best[n]:
            n += 1
        toks[s, :n] = drafts[s, :n]
        toks[s, n] = best[n]
        nacc[s] = n
    return toks, nacc


def test_greedy_onehot_ties_to_lowest_index():
    row = np.array([1.0, 3.0, -2.0, 3.0, 2.5], np.float32)
    p = oracle.distribution(row, LOGITS, 0.0)
    assert p.tolist() == [0.0, 1.0, 0.0, 0.0, 0.0]
    assert np.array_equal(oracle.distribution(row, LOGITS, -0.0), p)
    assert np.array_equal(oracle.greedy_onehot(row), p)
    assert oracle.distribution(row, LOGITS, 1.0).argmax() == 1 and oracle.distribution(row, LOGITS, 1.0)[0] > 0


def test_greedy_is_prefix_match():
    """T_p = 0: for any q (softmax, greedy or given probabilities) and any
    uniforms, the output is the longest prefix of drafts that agree with the
    target's largest logit, then the largest logit at the first disagreement
    (or of row K).  Small integer logits make ties common."""
    rng = np.random.default_rng(21)
    S, K, V = 60, 4, 12
    tl = rng.integers(-3, 4, size=(S * (K + 1), V)).astype(np.float32)
    dl = rng.normal(size=(S * K, V)).astype(np.float32)
    drafts = rng.integers(0, V, size=(S, K)).astype(np.int32)
    agree = rng.random((S, K)) < 0.75
    for s in range(S):
        for i in range(K):
            if agree[s, i]:
                drafts[s, i] = _first_max(tl[s * (K + 1) + i])
    u = rng.random((S, K + 1)).astype(np.float32)
    want_t, want_n = _prefix_match(tl, drafts, S, K)
    assert set(want_n.tolist()) == set(range(K + 1))
    qp = np.abs(dl) + 0.01
    qp = (qp / qp.sum(1, keepdims=True)).astype(np.float32)
    for draft, dk, t_q in ((dl, LOGITS, 1.0), (dl, LOGITS, 0.0), (qp, PROBS, 1.0)):
        toks, nacc = oracle.spec_accept(S, K, V, tl, LOGITS, 0.0, draft, dk, t_q, drafts, u)
        assert np.array_equal(nacc, want_n) and np.array_equal(toks, want_t)


def test_greedy_is_the_low_temperature_limit():
    """Distinct integer logits (gaps of at least 1): at T = 0.01 the softmax
    puts all but e^-100 of the mass on the maximum, so with uniforms away
    from 0 the outputs at T = 0.01 and at T = 0 agree, for both p and q."""
    rng = np.random.default_rng(22)
    S, K, V = 30, 3, 16
    tl = np.stack([rng.permutation(V) for _ in range(S * (K + 1))]).astype(np.float32)
    dl = np.stack([rng.permutation(V) for _ in range(S * K)]).astype(np.float32)
    drafts = np.where(rng.random((S, K)) < 0.7, tl.reshape(S, K + 1, V)[:, :K].argmax(-1),
                      rng.integers(0, V, size=(S, K))).astype(np.int32)
    u = (0.01 + 0.98 * rng.random((S, K + 1))).astype(np.float32)
    # a greedy drafter drafts its own largest logit (elsewhere q(d) = 0, and
    # 0 < p(d) = e^-100 would accept at T = 0.01): its rows copy the target's
    # for 70 % of the positions
    same = rng.random((S * K, 1)) < 0.7
    dl0 = np.where(same, tl.reshape(S, K + 1, V)[:, :K].reshape(S * K, V), dl)
    drafts0 = dl0.argmax(-1).reshape(S, K).astype(np.int32)
    for t_q, q, d in ((1.0, dl, drafts), (0.0, dl0, drafts0)):
        cold = oracle.spec_accept(S, K, V, tl, LOGITS, 0.01, q, LOGITS, t_q, d, u)
        zero = oracle.spec_accept(S, K, V, tl, LOGITS, 0.0, q, LOGITS, t_q, d, u)
        assert np.array_equal(cold[0], zero[0]) and np.array_equal(cold[1], zero[1])
        assert set(zero[1].tolist()) >= {0, K}
    # q greedy, p soft: the draft is q's largest logit, accepted iff u < p(d)
    d = int(dl[0].argmax())
    p_rows = [oracle.softmax_t(tl[i], 1.0) for i in range(K + 1)]
    q_rows = [oracle.distribution(dl[i], LOGITS, 0.0) for i in range(K)]
    for uu in (0.0, float(p_rows[0][d]) * 0.999, float(p_rows[0][d]) * 1.001):
        n, _ = oracle.accept_sequence(p_rows, q_rows, [d] + [0] * (K - 1), [uu] + [0.5] * K)
        assert (n >= 1) == (uu < p_rows[0][d])
