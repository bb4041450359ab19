"""Pins of the oracle's target-sample matching rule and of the yield-quench
accounting (CPU only).

Target-sample matching: hand-worked runs (tests/golden/target_sample_v4.json),
exact enumeration of the emitted-token distribution on tiny vocabularies (it
must equal the target distribution whatever the draft distribution), the
first-draft acceptance sum_x q(x) p(x), the K = 0 and greedy special cases.
The accounting: closed forms for a constant number of tokens per step, the
strict threshold on exactly representable values, skipped invalid steps and
banked credit.
"""
import itertools
import json
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
    for c in json.load(open(os.path.join(GOLDEN, "target_sample_v4.json")))["cases"]:
        p = [[F(v) for v in row] for row in c["p"]]
        u = [F(v) for v in c["u"]]
        assert oracle.target_sample_sequence(p, c["drafts"], u) == (c["n_accepted"], c["tokens"]), c["name"]
        # the fp64 path agrees (every u * Z and running sum here is exact in fp64)
        pn = [np.array([float(v) for v in row]) for row in p]
        got = oracle.target_sample_sequence(pn, c["drafts"], [float(v) for v in u])
        assert got == (c["n_accepted"], c["tokens"]), c["name"]


def _rand_dist(rng, V, zero_prob):
    while True:
        w = [0 if rng.random() < zero_prob else rng.randint(1, 9) for _ in range(V)]
        if sum(w):
            return [F(x, sum(w)) for x in w]


def _cells(w):
    """[(x, lo, hi)]: u in [lo, hi) picks x by the first-exceeding rule."""
    z = sum(w)
    out, c = [], F(0)
    for x, wx in enumerate(w):
        if wx > 0:
            out.append((x, c / z, (c + wx) / z))
        c += wx
    return out


def _enumerate(V, K, p_tab, q_tab):
    """Emitted-prefix distribution of the oracle, driven with the midpoint of
    every cell of every row it reads (and each cell's lower edge, which the
    strict rule gives to the same token)."""
    dist = {}
    for drafts in itertools.product(range(V), repeat=K):
        wq = F(1)
        for i in range(K):
            wq *= q_tab[drafts[:i]][drafts[i]]
        if wq == 0:
            continue
        p_rows = [p_tab[drafts[:i]] for i in range(K + 1)]

        def walk(i, us, prob):
            for x, lo, hi in _cells(p_rows[i]):
                u = us + [(lo + hi) / 2]
                if i < K and x == drafts[i]:
                    walk(i + 1, u, prob * (hi - lo))
                    continue
                pad = [F(0)] * (K + 1 - len(u))
                want = list(drafts[:i]) + [x]
                assert oracle.target_sample_sequence(p_rows, list(drafts), u + pad) == (i, want)
                assert oracle.target_sample_sequence(p_rows, list(drafts), us + [lo] + pad)[1] == want
                key = tuple(want)
                dist[key] = dist.get(key, F(0)) + prob * (hi - lo)

        walk(0, [], wq)
    return dist


@pytest.mark.parametrize("V,K", [(2, 1), (2, 3), (3, 1), (3, 2), (4, 1), (4, 2), (4, 3)])
def test_exact_enumeration_lossless(V, K):
    rng = random.Random(7000 + 10 * V + K)
    for _ in range(3 if V * K > 8 else 6):
        prefixes = [pre for L in range(K + 1) for pre in itertools.product(range(V), repeat=L)]
        p_tab = {pre: _rand_dist(rng, V, 0.25) for pre in prefixes}
        q_tab = {pre: _rand_dist(rng, V, 0.25) for pre in prefixes}
        dist = _enumerate(V, K, p_tab, q_tab)
        assert sum(dist.values()) == 1
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
            want = F(1)
            for j in range(K + 1):
                want *= p_tab[seq[:j]][seq[j]]
            assert full.get(seq, F(0)) == want, (seq, full.get(seq), want)


def test_first_draft_acceptance_is_sum_qp():
    """A draft d drawn from q stands with probability p(d), so the first-draft
    acceptance is sum_x q(x) p(x) (at most the p/q rule's 1 - TV)."""
    rng = random.Random(11)
    for _ in range(20):
        V = 5
        p, q = _rand_dist(rng, V, 0.2), _rand_dist(rng, V, 0.2)
        acc = F(0)
        for d in range(V):
            stand = sum(hi - lo for x, lo, hi in _cells(p) if x == d)
            for x, lo, hi in _cells(p):
                n, _ = oracle.target_sample_sequence([p, p], [d], [(lo + hi) / 2, F(0)])
                assert (n == 1) == (x == d)
            acc += q[d] * stand
        assert acc == sum(a * b for a, b in zip(p, q))
        assert acc <= sum(min(a, b) for a, b in zip(p, q))


def test_no_drafts_is_the_plain_sample():
    """K = 0: the step is one sample of row 0, the same as the p/q rule's
    bonus sample with the same uniform."""
    rng = np.random.default_rng(3)
    S, V = 40, 50
    tl = rng.normal(size=(S, V)).astype(np.float32)
    u = rng.random((S, 1)).astype(np.float32)
    empty = np.zeros((S, 0), np.int32)
    a = oracle.spec_accept_target_sample(S, 0, V, tl, LOGITS, 0.9, empty, u)
    b = oracle.spec_accept(S, 0, V, tl, LOGITS, 0.9, None, LOGITS, 1.0, empty, u)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert np.all(a[1] == 0)


def _first_max(row):
    vals = [float(v) for v in row]
    return vals.index(max(vals))


def test_greedy_is_prefix_match():
    """T_p = 0: the longest prefix of drafts equal to their rows' first
    largest logits, then the next row's first largest logit, for any
    uniforms (written without the rule)."""
    rng = np.random.default_rng(23)
    S, K, V = 60, 4, 12
    tl = rng.integers(-3, 4, size=(S * (K + 1), V)).astype(np.float32)
    drafts = rng.integers(0, V, size=(S, K)).astype(np.int32)
    agree = rng.random((S, K)) < 0.75
    for s in range(S):
        for i in range(K):
            if agree[s, i]:
                drafts[s, i] = _first_max(tl[s * (K + 1) + i])
    u = rng.random((S, K + 1)).astype(np.float32)
    toks, nacc = oracle.spec_accept_target_sample(S, K, V, tl, LOGITS, 0.0, drafts, u)
    for s in range(S):
        best = [_first_max(tl[s * (K + 1) + i]) for i in range(K + 1)]
        n = 0
        while n < K and int(drafts[s][n]) == best[n]:
            n += 1
        assert nacc[s] == n
        assert toks[s].tolist() == list(drafts[s, :n]) + [best[n]] + [-1] * (K - n)
    assert set(nacc.tolist()) == set(range(K + 1))


def test_batched_form_and_invalid_inputs():
    rng = np.random.default_rng(5)
    S, K, V = 5, 3, 9
    tl = rng.normal(size=(S * (K + 1), V)).astype(np.float32) * 2
    drafts = rng.integers(0, V, size=(S, K)).astype(np.int32)
    u = rng.random(size=(S, K + 1)).astype(np.float32)
    toks, nacc = oracle.spec_accept_target_sample(S, K, V, tl, LOGITS, 1.0, drafts, u)
    for s in range(S):
        p_rows = [oracle.softmax_t(tl[s * (K + 1) + i], 1.0) for i in range(K + 1)]
        n, out = oracle.target_sample_sequence(p_rows, drafts[s].tolist(), [float(x) for x in u[s]])
        assert nacc[s] == n and toks[s, :n + 1].tolist() == out and np.all(toks[s, n + 1:] == -1)
        # every emitted token is row j's own sample with uniform j
        for j in range(n + 1):
            assert toks[s, j] == oracle.first_exceeding(p_rows[j], float(u[s, j]))
    bad = [drafts.copy(), u.copy(), tl.copy()]
    bad[0][1, 0] = -1
    bad[1][2, 3] = 1.0
    bad[2][3 * (K + 1) + 2, 5] = np.inf
    outs = [oracle.spec_accept_target_sample(S, K, V, tl, LOGITS, 1.0, bad[0], u),
            oracle.spec_accept_target_sample(S, K, V, tl, LOGITS, 1.0, drafts, bad[1]),
            oracle.spec_accept_target_sample(S, K, V, bad[2], LOGITS, 1.0, drafts, u)]
    for (t, n), s_bad in zip(outs, (1, 2, 3)):
        assert n[s_bad] == -1 and np.all(t[s_bad] == -1)
        keep = [s for s in range(S) if s != s_bad]
        assert np.array_equal(n[keep], nacc[keep]) and np.array_equal(t[keep], toks[keep])
    pr = np.abs(rng.normal(size=(S * (K + 1), V))).astype(np.float32)
    pr[4 * (K + 1) + 1] = 0.0
    t4, n4 = oracle.spec_accept_target_sample(S, K, V, pr, PROBS, 1.0, drafts, u)
    assert n4[4] == -1 and np.all(n4[:4] >= 0)


# ------------------------------------------------------------ accounting

def test_quench_constant_tokens_closed_form():
    """t tokens every step: regret after k steps is k (g - t), so the quench
    falls at the first k with k (g - t) > th, k = floor(th / (g - t)) + 1,
    and never when t >= g (exact arithmetic)."""
    g, th = F(54, 25), F(4)          # 2.16 and 4
    for t in range(1, 6):
        n = t - 1
        steps, tokens, regret, q = oracle.yield_quench([n] * 50, g, th)
        if t >= g:
            assert q is None and steps == 50 and tokens == 50 * t and regret == 50 * (g - t)
        else:
            k = int(th // (g - t)) + 1
            assert q == k and steps == k and tokens == k * t and regret == k * (g - t)


def test_quench_threshold_is_strict():
    g, th = F(9, 4), F(4)            # regret 1.25 per one-token step
    # 1.25, 2.5, 3.75, 5.0: quenched at step 4
    assert oracle.yield_quench([0] * 10, g, th)[3] == 4
    # reach exactly 4: 1.25 * 2 + (2.25 - 1) ... use t = 2 steps (0.25 each): 16 steps give 4.0
    r = oracle.yield_quench([1] * 16, g, th)
    assert r[2] == 4 and r[3] is None
    assert oracle.yield_quench([1] * 17, g, th)[3] == 17
    # the same in fp64 (every value exact)
    assert oracle.yield_quench([1] * 16, 2.25, 4.0)[3] is None
    assert oracle.yield_quench([1] * 17, 2.25, 4.0)[3] == 17


def test_quench_skips_invalid_and_banks_credit():
    g, th = F(54, 25), F(4)
    # invalid steps (-1) commit nothing and are not counted
    a = oracle.yield_quench([0, -1, 0, -1, 0], g, th)
    b = oracle.yield_quench([0, 0, 0], g, th)
    assert a == b and a[0] == 3 and a[1] == 3
    # five-token steps bank 2.84 each; two of them cover three one-token steps
    # (3 * 1.16 = 3.48 < 5.68) plus up to threshold
    seq = [4, 4] + [0] * 8
    steps, tokens, regret, q = oracle.yield_quench(seq, g, th)
    # regret: -5.68 + k * 1.16 > 4 first at k = 9 (10.44 - 5.68 = 4.76), i.e. never within 8
    assert q is None and regret == 2 * (g - 5) + 8 * (g - 1)
    steps, tokens, regret, q = oracle.yield_quench([4, 4] + [0] * 9, g, th)
    assert q == 11 and steps == 11 and tokens == 19
    # later steps after the quench are not counted
    assert oracle.yield_quench([0] * 4 + [4] * 10, g, th)[:2] == (4, 4)


def test_quench_hand_worked():
    """guard 2.16, threshold 4; steps committing 3, 1, 1, 2, 1, 1, 1, 1 tokens:
    regret -0.84, 0.32, 1.48, 1.64, 2.80, 3.96, 5.12 -> quenched at step 7
    (3.96 does not exceed 4)."""
    g, th = F(54, 25), F(4)
    steps, tokens, regret, q = oracle.yield_quench([2, 0, 0, 1, 0, 0, 0, 0], g, th)
    assert (steps, tokens, q) == (7, 10, 7) and regret == F(512, 100)
