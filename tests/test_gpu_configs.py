"""GPU parity at the full sizes of the five workloads, in the launch
configuration the benchmark times, on outputs the oracle computes one by one.

* one SwiGLU expert (7168 -> 2048 -> 7168, two-bit) on R = 1, 2, 4, 8 bf16
  rows: every output against the oracle;
* the full MoE layer (256 routed + 1 shared experts, top-8) on R = 5 rows:
  routing indices bit-exact for every row, routing weights and every row of y
  against the oracle;
* the vocabulary head (129,280 x 7,168, eight-bit) on R = 5 rows: every logit
  against the oracle, then spec_accept at V = 129,280 and T = 0.8 on the GPU's
  logits (T_q = 0.8 and the T_q = 1 variant), decisions compared with the
  oracle's on identical inputs;
* the cohort: 3 sequences x 5 rows = 15 rows through the same layer (every row
  of y against the oracle) and head, per-sequence spec_accept;
* run-to-run determinism: the layer, the head and spec_accept repeated on the
  same inputs give bit-identical outputs;
* the R = 1..16 stress sweep: every R against the oracle on sampled vocabulary
  rows, and every row of every R-row MoE call against the oracle (the routing
  bit-exact; the expert sums may round differently with the batch, since an
  expert's rows are contracted one way when it has one row and another when
  it has several);
* a full-vocabulary rejection workload given as probabilities, where decisions
  and tokens must match the oracle exactly (identical fp32 p, q and u).
* the eight-bit router GEMV ([256 x 7168], through the head's call) ahead of
  the layer: every logit against the oracle, then the routing bit-exact on the
  GPU's logits;
* target-sample matching at V = 129,280 on the head's own logits (the cohort
  shape, 3 sequences x 4 drafts, and one sequence of 15 drafts).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.accept import LOGITS, PROBS
from tests.gpu_util import dev, empty, host, say
from tests.parity import (accept_flags, assert_close, check_target_sample, matching_drafts,
                          sample_flag)

pytestmark = pytest.mark.gpu

H, I, V, E, TOPK = synth.HIDDEN, synth.INTER, synth.VOCAB, synth.N_ROUTED, synth.TOP_K
BG = oracle.q2_matrix_bytes(I, H)
BD = oracle.q2_matrix_bytes(H, I)


@pytest.fixture(scope="module")
def sv():
    import bit_moe_tiny_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def layer(sv):
    """The MoE layer of the moe_layer workload, resident on the GPU, plus the
    host buffers the oracle reads."""
    say("generating the MoE layer (257 experts)")
    w = synth.moe_weights(synth.CFG_MOE)
    t = [dev(a) for a in (w.gate, w.up, w.down, w.s_gate, w.s_up, w.s_down)]
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, H, I, E, TOPK, *t)
    return w, desc


@pytest.fixture(scope="module")
def head(sv):
    say("generating the vocabulary head")
    buf = synth.lm_head_weights().packed()
    return buf, dev(buf)


def _vocab_sample(seed: int, n: int = 2048) -> np.ndarray:
    rng = np.random.default_rng(seed)
    pick = rng.choice(V, size=n, replace=False)
    return np.unique(np.concatenate([np.arange(64), np.arange(V - 64, V), pick]))


def _oracle_moe_rows(w, x_bf16, logits, rows):
    """Oracle y for the given rows only (each row's output depends on that row alone)."""
    sub_x = x_bf16[rows]
    sub_l = logits[rows]
    y, idx, wts = oracle.moe_layer(w.gate, w.up, w.down, w.s_gate, w.s_up, w.s_down, E, TOPK, H,
                                   I, sub_x, "bf16", sub_l)
    return y


def _run_moe(sv, desc, x, logits):
    R = x.shape[0]
    y = empty((R, H), "f32")
    ti = empty((R, TOPK), "i32")
    tw = empty((R, TOPK), "f32")
    sv.vq2_moe_gemm(desc, dev(x), dev(logits), y, ti, tw)
    return host(y), host(ti), host(tw)


def _run_head(sv, wdev, h):
    R = h.shape[0]
    z = empty((R, V), "f32")
    sv.vq8_lmhead_gemm(wdev, V, H, dev(h), z)
    return host(z)


def _check_accept(sv, z, S, K, Tp, Tq, acc):
    """spec_accept on the GPU vs the oracle on the same fp32 logits."""
    toks = empty((S, K + 1), "i32")
    nacc = empty((S,), "i32")
    say("spec_accept", S, K, V, Tp, Tq)
    sv.spec_accept(S, K, V, dev(z), sv.SV_LOGITS, Tp, dev(acc.draft_logits), sv.SV_LOGITS, Tq,
                   dev(acc.drafts), dev(acc.uniforms), toks, nacc)
    gt, gn = host(toks), host(nacc)
    wt, wn = oracle.spec_accept(S, K, V, z, LOGITS, Tp, acc.draft_logits, LOGITS, Tq, acc.drafts,
                                acc.uniforms)
    zz = z.reshape(S, K + 1, V)
    dd = acc.draft_logits.reshape(S, K, V)
    for s in range(S):
        p_rows = [oracle.softmax_t(zz[s, i], Tp) for i in range(K + 1)]
        q_rows = [oracle.softmax_t(dd[s, i], Tq) for i in range(K)]
        if accept_flags(p_rows, q_rows, acc.drafts[s], acc.uniforms[s], int(wn[s])):
            continue   # an accept test within 1e-6 of its boundary: flagged, not failed
        assert gn[s] == wn[s], f"sequence {s}: n_accepted {gn[s]} vs oracle {wn[s]}"
        n = int(wn[s])
        if not np.array_equal(gt[s], wt[s]):
            wgt = (np.maximum(p_rows[n] - q_rows[n], 0.0) if n < K else p_rows[K])
            assert sample_flag(wgt, acc.uniforms[s, K]), (
                f"sequence {s}: tokens {gt[s]} vs oracle {wt[s]}")
    return wn


# ---------------------------------------------------------------- expert
@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_expert_workload(sv, R):
    ex = synth.expert(R)
    g, u, d = (ex.mats[m].packed() for m in (synth.M_GATE, synth.M_UP, synth.M_DOWN))
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, H, I, 1, 1, dev(g), dev(u), dev(d))
    y = empty((R, H), "f32")
    say("vq2_moe_gemm one expert", R)
    sv.vq2_moe_gemm(desc, dev(ex.x_bf16), None, y)
    x64 = oracle.linalg._exact_rows(ex.x_bf16, "bf16")
    want = oracle.swiglu_expert(g, u, d, H, I, x64)
    assert_close(host(y), want, what=f"one expert R={R} y (every output)")


# ------------------------------------------------------------- MoE layer
def test_moe_layer_workload(sv, layer):
    w, desc = layer
    rows = synth.moe_rows(5, synth.CFG_MOE)
    say("vq2_moe_gemm full layer R=5")
    y, ti, tw = _run_moe(sv, desc, rows.x_bf16, rows.router_logits)
    widx, ww = oracle.route_topk(rows.router_logits, TOPK)
    assert np.array_equal(ti, widx)
    assert_close(tw, ww, what="moe layer R=5 topk_w")
    say("oracle MoE output, all 5 rows")
    want = _oracle_moe_rows(w, rows.x_bf16, rows.router_logits, list(range(5)))
    assert_close(y, want, what="moe layer R=5 y (every row)")


@pytest.mark.parametrize("R", [5, 16])
def test_moe_layer_eight_bit_shared(sv, layer, R):
    """The full layer with its shared expert in eight-bit blocks (the
    format of the pages' model): the 256 routed experts of the workload, an
    eight-bit shared expert of the same shape; every row of y against the
    oracle."""
    w, _ = layer
    say("eight-bit shared expert, layer R =", R)
    sq = [m.packed() for m in synth.shared_q8_weights()]
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, H, I, E, TOPK, *(dev(a) for a in (w.gate, w.up, w.down)),
                       *(dev(a) for a in sq), shared_format=sv.SV_Q8)
    rows = synth.moe_rows(R, synth.CFG_MOE, sub=40 + R)
    y, ti, _ = _run_moe(sv, desc, rows.x_bf16, rows.router_logits)
    widx, _ = oracle.route_topk(rows.router_logits, TOPK)
    assert np.array_equal(ti, widx)
    say("oracle MoE output with the eight-bit shared expert, all rows")
    want, _, _ = oracle.moe_layer(w.gate, w.up, w.down, *sq, E, TOPK, H, I, rows.x_bf16, "bf16",
                                  rows.router_logits, shared_format="q8")
    assert_close(y, want, what=f"moe layer q8 shared R={R} y (every row)")


# ---------------------------------------------------------------- router
def test_router_gemv_then_layer(sv, layer):
    """The eight-bit router GEMV ahead of the top-k, as the vocabulary head's
    call on a [256 x 7168] matrix: every logit against the oracle, then the
    layer on the GPU's fp32 logits, its routing bit-exact against the oracle's
    top-k of the same logits (the decision taken in the same precision on
    both sides), and two rows of y against the oracle."""
    w, desc = layer
    rows = synth.moe_rows(5, synth.CFG_MOE)
    wr = synth.router_weights().packed()
    R = rows.x_bf16.shape[0]
    z = empty((R, E), "f32")
    say("vq8_lmhead_gemm router GEMV [256 x 7168] R=5")
    sv.vq8_lmhead_gemm(dev(wr), E, H, dev(rows.x_bf16), z)
    z = host(z)
    assert_close(z, oracle.lm_head_logits(wr, E, H, rows.x_bf16, "bf16"), what="router GEMV logits [256 x 7168] R=5")
    say("vq2_moe_gemm on the router GEMV's logits R=5")
    y, ti, tw = _run_moe(sv, desc, rows.x_bf16, z)
    widx, ww = oracle.route_topk(z, TOPK)
    assert np.array_equal(ti, widx)
    assert_close(tw, ww, what="router GEMV R=5 topk_w")
    assert len(np.unique(ti)) > 2 * TOPK   # the rows route to different experts
    say("oracle MoE output on the router GEMV's logits, all 5 rows")
    assert_close(y, _oracle_moe_rows(w, rows.x_bf16, z, list(range(R))),
                 what="moe layer R=5 y on router GEMV logits (every row)")


# ------------------------------------------------------------ vocab head
@pytest.mark.parametrize("Tq", [0.8, 1.0])
def test_lm_head_workload_and_accept(sv, head, Tq):
    buf, wdev = head
    R, S, K, T = 5, 1, 4, 0.8
    h = synth.lm_head_hidden(R)
    say("vq8_lmhead_gemm full head R=5")
    z = _run_head(sv, wdev, h)
    say("oracle head, every logit")
    want = oracle.lm_head_logits(buf, V, H, h, "bf16")
    assert_close(z, want, what=f"lm head R=5 (every logit, T_q={Tq} case)")
    acc = synth.accept_inputs(z, S, K, 1.5, Tq, synth.CFG_LMHEAD)
    _check_accept(sv, z, S, K, T, Tq, acc)


def test_lm_head_greedy(sv, head):
    """Greedy decoding (T_p = T_q = 0) on the head's own logits at
    V = 129,280, drafts from a greedy drafter (its largest draft logit): exact
    against the oracle and against the prefix-match form."""
    buf, wdev = head
    R, S, K = 5, 1, 4
    say("vq8_lmhead_gemm full head R=5, greedy spec_accept")
    z = _run_head(sv, wdev, synth.lm_head_hidden(R))
    acc = synth.accept_inputs(z, S, K, 0.3, 1.0, synth.CFG_LMHEAD, sub=7)
    drafts = acc.draft_logits.reshape(S, K, V).argmax(-1).astype(np.int32)
    toks = empty((S, K + 1), "i32")
    nacc = empty((S,), "i32")
    sv.spec_accept(S, K, V, dev(z), sv.SV_LOGITS, 0.0, dev(acc.draft_logits), sv.SV_LOGITS, 0.0,
                   dev(drafts), dev(acc.uniforms), toks, nacc)
    toks, nacc = host(toks), host(nacc)
    wt, wn = oracle.spec_accept(S, K, V, z, LOGITS, 0.0, acc.draft_logits, LOGITS, 0.0, drafts,
                                acc.uniforms)
    assert np.array_equal(nacc, wn) and np.array_equal(toks, wt)
    best = z.argmax(-1)
    n = 0
    while n < K and drafts[0, n] == best[n]:
        n += 1
    assert nacc[0] == n and toks[0, :n].tolist() == drafts[0, :n].tolist() and toks[0, n] == best[n]


# ---------------------------------------------------------------- cohort
def test_cohort_workload(sv, layer, head):
    w, desc = layer
    buf, wdev = head
    R, S, K, T = 15, 3, 4, 0.8
    rows = synth.moe_rows(R, synth.CFG_COHORT)
    say("vq2_moe_gemm cohort R=15")
    y, ti, tw = _run_moe(sv, desc, rows.x_bf16, rows.router_logits)
    widx, ww = oracle.route_topk(rows.router_logits, TOPK)
    assert np.array_equal(ti, widx)
    assert_close(tw, ww, what="cohort R=15 topk_w")
    say("oracle MoE output, all 15 cohort rows")
    assert_close(y, _oracle_moe_rows(w, rows.x_bf16, rows.router_logits, list(range(R))),
                 what="cohort R=15 moe y (every row)")
    h = synth.lm_head_hidden(R, synth.CFG_COHORT)
    say("vq8_lmhead_gemm cohort R=15")
    z = _run_head(sv, wdev, h)
    cols = _vocab_sample(32, 1024)
    assert_close(z[:, cols], oracle.lm_head_logits(buf, V, H, h, "bf16", rows=cols),
                 what="cohort head R=15 (1,024 sampled vocabulary rows)")
    acc = synth.accept_inputs(z, S, K, 1.5, T, synth.CFG_COHORT)
    _check_accept(sv, z, S, K, T, T, acc)


# ----------------------------------------------------------------- sweep
@pytest.fixture(scope="module")
def sweep16(sv, layer, head):
    """16-row inputs of the sweep, the GPU results of the 16-row calls and the
    oracle's MoE output for all 16 rows."""
    w, desc = layer
    buf, wdev = head
    rows = synth.moe_rows(16, synth.CFG_COHORT, sub=16)
    h = synth.lm_head_hidden(16, synth.CFG_COHORT, sub=16)
    say("sweep reference calls R=16")
    y16, ti16, _ = _run_moe(sv, desc, rows.x_bf16, rows.router_logits)
    z16 = _run_head(sv, wdev, h)
    say("oracle MoE output of the 16 sweep rows")
    y_or = _oracle_moe_rows(w, rows.x_bf16, rows.router_logits, list(range(16)))
    return rows, h, y16, ti16, z16, y_or


def test_sweep_moe_r16_against_oracle(sv, layer, sweep16):
    rows, _, y16, ti16, _, y_or = sweep16
    assert np.array_equal(ti16, oracle.route_topk(rows.router_logits, TOPK)[0])
    assert_close(y16, y_or, what="sweep R=16 moe y")


@pytest.mark.parametrize("R", list(range(1, 16)))
def test_sweep_moe_rows(sv, layer, sweep16, R):
    """Every row of an R-row call against the oracle; the routing of row r
    equals that of the 16-row call (it depends on that row alone)."""
    _, desc = layer
    rows, _, _, ti16, _, y_or = sweep16
    say("vq2_moe_gemm sweep", R)
    y, ti, _ = _run_moe(sv, desc, rows.x_bf16[:R].copy(), rows.router_logits[:R].copy())
    assert np.array_equal(ti, ti16[:R])
    assert_close(y, y_or[:R], what=f"sweep moe R={R} y (every row)")


@pytest.mark.parametrize("R", list(range(1, 17)))
def test_sweep_lm_head(sv, head, sweep16, R):
    buf, wdev = head
    _, h, _, _, z16, _ = sweep16
    say("vq8_lmhead_gemm sweep", R)
    z = _run_head(sv, wdev, h[:R].copy())
    cols = _vocab_sample(100 + R, 512)
    assert_close(z[:, cols], oracle.lm_head_logits(buf, V, H, h[:R], "bf16", rows=cols),
                 what=f"sweep head R={R} (512 sampled vocabulary rows)")
    assert_close(z, z16[:R], tol=1e-5, what=f"head R={R} vs R=16")


@pytest.mark.parametrize("S,K,T", [(3, 4, 0.8), (1, 15, 1.0)])
def test_target_sample_full_vocab(sv, sweep16, S, K, T):
    """Target-sample matching on the head's 16 logit rows of the sweep
    (V = 129,280), drafts equal to the target's own sample 70 % of the time:
    outputs against the oracle on the same logits."""
    z = sweep16[4][:S * (K + 1)]
    g = synth.generator(160, S, K)
    u = synth.uniform24(g, S * (K + 1)).reshape(S, K + 1)
    drafts = matching_drafts(S, K, V, z, LOGITS, T, u, 0.7, np.random.default_rng(160 + K))
    toks = empty((S, K + 1), "i32")
    nacc = empty((S,), "i32")
    say("spec_accept_target_sample full vocab", S, K, T)
    sv.spec_accept_target_sample(S, K, V, dev(z), sv.SV_LOGITS, T, dev(drafts), dev(u), toks, nacc)
    wn, flagged = check_target_sample(S, K, V, z, LOGITS, T, drafts, u, host(toks), host(nacc))
    assert np.all(wn >= 0) and flagged == 0


# ----------------------------------------------- full-vocabulary rejection
@pytest.mark.parametrize("S,K", [(4, 4), (2, 0), (1, 15)])
def test_full_vocab_probs_exact(sv, S, K):
    """p and q over V = 129,280 given as fp32 probabilities (q a perturbed p,
    so rejections happen): decisions bit-exact, tokens exact unless the
    sampling target sits on a CDF boundary."""
    g = synth.generator(120, S, K)
    zt = synth.normal(g, S * (K + 1) * V, 2.0).reshape(S * (K + 1), V)
    p = np.stack([oracle.softmax_t(r.astype(np.float32), 1.0) for r in zt]).astype(np.float32)
    q = np.zeros((0, V), np.float32)
    drafts = np.zeros((S, K), np.int32)
    if K:
        zq = (zt.reshape(S, K + 1, V)[:, :K].reshape(S * K, V)
              + synth.normal(g, S * K * V, 1.5).reshape(S * K, V))
        q = np.stack([oracle.softmax_t(r.astype(np.float32), 1.0) for r in zq]).astype(np.float32)
        drafts = synth.gumbel_drafts(zq.astype(np.float32), 1.0, g).reshape(S, K)
    u = synth.uniform24(g, S * (K + 1)).reshape(S, K + 1)
    toks = empty((S, K + 1), "i32")
    nacc = empty((S,), "i32")
    say("spec_accept probs full vocab", S, K)
    sv.spec_accept(S, K, V, dev(p), sv.SV_PROBS, 1.0, dev(q) if K else None, sv.SV_PROBS, 1.0,
                   dev(drafts) if K else None, dev(u), toks, nacc)
    gt, gn = host(toks), host(nacc)
    wt, wn = oracle.spec_accept(S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u)
    assert np.array_equal(gn, wn)
    for s in range(S):
        if np.array_equal(gt[s], wt[s]):
            continue
        n = int(wn[s])
        pr = p[s * (K + 1) + n].astype(np.float64)
        wgt = np.maximum(pr - q[s * K + n], 0.0) if n < K else pr
        assert sample_flag(wgt, u[s, K]), f"sequence {s}: {gt[s]} vs {wt[s]}"


# ----------------------------------------------------------- determinism
def test_repeat_bit_identical(sv, layer, head):
    """The three calls, repeated on the same inputs, give the same bits (every
    summation order is fixed; no atomics decide a floating-point order)."""
    _, desc = layer
    _, wdev = head
    R, S, K, T = 5, 1, 4, 0.8
    rows = synth.moe_rows(R, synth.CFG_MOE)
    h = synth.lm_head_hidden(R)
    say("determinism: layer, head and accept three times each")
    outs = []
    for _ in range(3):
        y, ti, tw = _run_moe(sv, desc, rows.x_bf16, rows.router_logits)
        z = _run_head(sv, wdev, h)
        outs.append((y, ti, tw, z))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))
    z = outs[0][3]
    acc = synth.accept_inputs(z, S, K, 1.5, T, synth.CFG_LMHEAD)
    res = []
    for _ in range(3):
        toks = empty((S, K + 1), "i32")
        nacc = empty((S,), "i32")
        sv.spec_accept(S, K, V, dev(z), sv.SV_LOGITS, T, dev(acc.draft_logits), sv.SV_LOGITS, T,
                       dev(acc.drafts), dev(acc.uniforms), toks, nacc)
        res.append((host(toks), host(nacc)))
    for r in res[1:]:
        assert np.array_equal(r[0], res[0][0]) and np.array_equal(r[1], res[0][1])
