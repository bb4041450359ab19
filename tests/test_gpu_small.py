"""GPU parity at sizes the oracle finishes in seconds: dequantisation
(bit-exact), the one-matrix two-bit product (the tiny configuration and ragged
shapes), a small routed MoE layer, a small vocabulary head, and the accept
rule on the tiny configuration.  Every call goes through the C ABI."""
import numpy as np
import pytest

import oracle
import synth
from oracle.accept import LOGITS, PROBS
from tests.gpu_util import dev, empty, host, say
from tests.parity import (accept_flags, assert_close, check_target_sample, matching_drafts,
                          sample_flag)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import bit_moe_tiny_amd as m
    m.load()
    return m


# ------------------------------------------------------------ dequant
@pytest.mark.parametrize("n,k", [(512, 256), (2048, 7168), (33, 768)])
def test_q2_dequant_bit_exact(sv, n, k):
    p = synth.q2_random(synth.generator(100, n, k), n, k, 0.02)
    buf = p.packed()
    say("vq2_dequant", n, k)
    out = empty((n, k), "f32")
    sv.vq2_dequant(dev(buf), n, k, out)
    got = host(out)
    want = oracle.q2_dequant_f32(buf, n, k)
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))
    if bad[0].size:
        q, sc, m, du, dmu = oracle.q2_fields(buf, n, k)
        rows, cols = bad
        info = [(int(r), int(c), int(q[r, c]), int(sc[r, c // 16]), int(m[r, c // 16]),
                 int(du[r, c // 256]), int(dmu[r, c // 256]), float(got[r, c]), float(want[r, c]))
                for r, c in list(zip(rows, cols))[:8]]
        pytest.fail(f"{rows.size} mismatches; (n,k,q,sc,m,d*2^24,dmin*2^24,got,want): {info}")


def _tiled_layout(buf, n, k, parts):
    """The expert-tiled layout as the header states it, written out with
    numpy loops from the plain planes (an independent restatement of the
    chunk formula, not a copy of the kernel's indexing)."""
    nb = k // 256
    nblk = n * nb
    up = lambda x: (x + 255) // 256 * 256
    qs = buf[:nblk * 64].reshape(n, nb, 64)
    o = up(nblk * 64)
    sc = buf[o:o + nblk * 16].reshape(n, nb, 16)
    o += up(nblk * 16)
    d = buf[o:o + nblk * 2].reshape(n, nb, 2)
    o += up(nblk * 2)
    dm = buf[o:o + nblk * 2].reshape(n, nb, 2)
    out = np.zeros(nblk * 84, np.uint8)
    for t in range(n // 16):
        rows = slice(16 * t, 16 * t + 16)
        for p in range(parts):
            b0, b1 = nb * p // parts, nb * (p + 1) // parts
            kb = b0
            while kb < b1:
                m = 1 if (kb % 2 or kb + 1 >= b1) else 2
                base = 1344 * (t * nb + kb)
                pieces = qs[rows, kb:kb + m].reshape(16, 4 * m, 16)
                for r in range(16):
                    for c in range(4 * m):
                        at = base + r * 64 * m + 16 * ((c + r) % (4 * m))
                        out[at:at + 16] = pieces[r, c]
                nib = sc[rows, kb:kb + m].reshape(16, m, 4, 4)          # [row][block][dword g][byte]
                out[base + 1024 * m:base + 1280 * m] = nib.transpose(1, 2, 0, 3).reshape(-1)
                out[base + 1280 * m:base + 1312 * m] = d[rows, kb:kb + m].reshape(-1)
                out[base + 1312 * m:base + 1344 * m] = dm[rows, kb:kb + m].reshape(-1)
                kb += m
    return out


@pytest.mark.parametrize("n,k,parts", [(32, 7168, 4), (16, 2048, 1), (32, 1792, 4), (48, 768, 4),
                                       (16, 2304, 1), (32, 2304, 3)])
def test_q2_tile_layout_bit_exact(sv, n, k, parts):
    """sv_q2_tile writes every byte where the documented chunk layout puts it
    (two matrices back to back: the second one's offset is checked too)."""
    mats = [synth.q2_random(synth.generator(109, n, k, i), n, k, 0.02).packed() for i in range(2)]
    say("sv_q2_tile", n, k, parts)
    got = host(sv.sv_q2_tile(dev(np.concatenate(mats)), n, k, parts, 2))
    want = np.concatenate([_tiled_layout(m, n, k, parts) for m in mats])
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8].tolist()}"


@pytest.mark.parametrize("n,k", [(777, 1024), (16, 7168)])
def test_q8_dequant_bit_exact(sv, n, k):
    p = synth.q8_random(synth.generator(101, n, k), n, k, 0.01)
    buf = p.packed()
    say("vq8_dequant", n, k)
    out = empty((n, k), "f32")
    sv.vq8_dequant(dev(buf), n, k, out)
    assert np.array_equal(host(out).view(np.uint32), oracle.q8_dequant_f32(buf, n, k).view(np.uint32))


# --------------------------------------------------------------- plain
def _plain(sv, buf, n_out, k_in, x):
    d = sv.moe_desc(sv.SV_FFN_PLAIN, k_in, n_out, 1, 1, dev(buf))
    y = empty((x.shape[0], n_out), "f32")
    sv.vq2_moe_gemm(d, x, None, y)
    return host(y)


def test_tiny_plain_layer(sv):
    t = synth.tiny()
    buf = t.w.packed()
    say("vq2_moe_gemm PLAIN tiny 512x256 R=4 f32")
    y = _plain(sv, buf, 512, 256, dev(t.x))
    want = oracle.plain_layer(buf, 512, 256, t.x, "f32")
    assert_close(y, want, what="tiny plain")


@pytest.mark.parametrize("n_out,k_in,R,dt", [(520, 768, 3, "f32"), (64, 256, 17, "bf16"),
                                            (1000, 1024, 33, "f32"), (7, 256, 1, "bf16")])
def test_plain_ragged(sv, n_out, k_in, R, dt):
    p = synth.q2_random(synth.generator(102, n_out, k_in), n_out, k_in, 0.02)
    buf = p.packed()
    g = synth.generator(103, R, k_in)
    x = synth.normal_bf16(g, (R, k_in)) if dt == "bf16" else synth.normal_f32(g, (R, k_in))
    say("vq2_moe_gemm PLAIN", n_out, k_in, R, dt)
    y = _plain(sv, buf, n_out, k_in, dev(x))
    want = oracle.plain_layer(buf, n_out, k_in, x, dt)
    assert_close(y, want, what=f"plain {n_out}x{k_in} R={R} {dt}")


# ----------------------------------------------------------------- MoE
def _small_moe(E, hidden, inter, shared, seed):
    mats = [synth.expert_matrices(seed, e, 0.02, hidden, inter) for e in range(E + (1 if shared else 0))]
    cat = lambda m: np.concatenate([mats[e][m].packed() for e in range(E)])
    ws = (cat(synth.M_GATE), cat(synth.M_UP), cat(synth.M_DOWN))
    sh = tuple(mats[E][m].packed() for m in (synth.M_GATE, synth.M_UP, synth.M_DOWN)) if shared else (None,) * 3
    return ws, sh


@pytest.mark.parametrize("E,k,hidden,inter,R,shared,dt", [
    (16, 4, 512, 256, 5, True, "bf16"),
    (8, 2, 256, 512, 3, False, "f32"),
    (32, 8, 1024, 256, 16, True, "bf16"),
    (4, 4, 256, 256, 20, True, "bf16"),
    (12, 3, 768, 1024, 7, True, "bf16"),    # down: 4 blocks per row, 6 row groups
    (6, 2, 1280, 1536, 9, True, "f32"),     # down: 6 blocks per row; shared expert in 3 column groups
    (2, 1, 256, 9216, 3, True, "f32"),      # down: 36 blocks per row, one row per column group
    (8, 2, 7168, 256, 6, True, "bf16"),     # gate/up: 28 blocks per row, parts of 4 and 3 blocks
    (4, 2, 8192, 512, 9, True, "f32"),      # gate/up: 32 blocks per row, parts of 4 blocks
    (20, 16, 256, 256, 64, True, "bf16"),   # the limits: R = 64 rows, top-16 of 20 experts
])
def test_small_moe_layer(sv, E, k, hidden, inter, R, shared, dt):
    (g, u, d), (sg, su, sd) = _small_moe(E, hidden, inter, shared, 104 + E)
    gen = synth.generator(105, E, R)
    x = synth.normal_bf16(gen, (R, hidden)) if dt == "bf16" else synth.normal_f32(gen, (R, hidden))
    logits = synth.normal_f32(synth.generator(106, E, R), (R, E))
    tens = [dev(a) if a is not None else None for a in (g, u, d, sg, su, sd)]
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, hidden, inter, E, k, *tens)
    y = empty((R, hidden), "f32")
    ti = empty((R, k), "i32")
    tw = empty((R, k), "f32")
    say("vq2_moe_gemm SWIGLU", E, k, hidden, inter, R, shared, dt)
    sv.vq2_moe_gemm(desc, dev(x), dev(logits), y, ti, tw)
    want, widx, ww = oracle.moe_layer(g, u, d, sg, su, sd, E, k, hidden, inter, x, dt, logits)
    assert np.array_equal(host(ti), widx)
    assert_close(host(tw), ww, what=f"small moe E={E} k={k} {hidden}x{inter} R={R} {dt} topk_w")
    assert_close(host(y), want, what=f"small moe E={E} k={k} {hidden}x{inter} R={R} shared={shared} {dt} y")


@pytest.mark.parametrize("E,k,hidden,inter,R,dt", [
    (16, 4, 512, 256, 5, "bf16"),
    (8, 2, 256, 512, 3, "f32"),
    (32, 8, 1024, 256, 16, "bf16"),
    (6, 2, 1280, 1536, 9, "f32"),
])
def test_small_moe_eight_bit_shared(sv, E, k, hidden, inter, R, dt):
    """The shared expert in eight-bit blocks (the head's kernels for its
    three products) beside two-bit routed experts."""
    (g, u, d), _ = _small_moe(E, hidden, inter, False, 107 + E)
    sq = synth.shared_q8_weights(108 + E, hidden, inter)
    sg, su, sd = (m.packed() for m in sq)
    gen = synth.generator(109, E, R)
    x = synth.normal_bf16(gen, (R, hidden)) if dt == "bf16" else synth.normal_f32(gen, (R, hidden))
    logits = synth.normal_f32(synth.generator(110, E, R), (R, E))
    tens = [dev(a) for a in (g, u, d, sg, su, sd)]
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, hidden, inter, E, k, *tens, shared_format=sv.SV_Q8)
    y = empty((R, hidden), "f32")
    ti = empty((R, k), "i32")
    say("vq2_moe_gemm SWIGLU eight-bit shared", E, k, hidden, inter, R, dt)
    sv.vq2_moe_gemm(desc, dev(x), dev(logits), y, ti)
    want, widx, _ = oracle.moe_layer(g, u, d, sg, su, sd, E, k, hidden, inter, x, dt, logits,
                                     shared_format="q8")
    assert np.array_equal(host(ti), widx)
    assert_close(host(y), want, what=f"small moe q8 shared E={E} k={k} {hidden}x{inter} R={R} {dt} y")


# ------------------------------------------------------------ routing ties
def _tie_logits(R, E, seed):
    """Router rows built to exercise the tie-breaking rule (equal logits: the
    lower index first), each kind of row twice:
    integer logits in -3..3 (the top value tied at many indices in every
    64-expert slot); all zeros with mixed signs except a few negatives (+0 and
    -0 tie); zeros of both signs planted at indices 3 (-0), 5 (+0), 69 (-0),
    132 (+0) and 200 (-0) among negatives; rows with -inf entries (fewer than
    k finite logits in one row), rows with NaN entries (NaN ranks last), a row
    with a +inf entry, and an all -inf row."""
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(2):
        rows.append(rng.integers(-3, 4, size=E).astype(np.float32))
        z = np.where(rng.random(E) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        z[rng.choice(E, 40, replace=False)] = -rng.random(40).astype(np.float32) - 0.5
        rows.append(z)
        z = -rng.random(E).astype(np.float32) - 1.0
        for i, v in ((3, -0.0), (5, 0.0), (69, -0.0), (132, 0.0), (200, -0.0)):
            z[i] = np.float32(v)
        rows.append(z)
        z = rng.integers(-2, 3, size=E).astype(np.float32)
        z[rng.choice(E, E - 5, replace=False)] = -np.inf
        rows.append(z)
        z = rng.integers(-2, 3, size=E).astype(np.float32)
        z[rng.choice(E, 60, replace=False)] = np.nan
        rows.append(z)
    z = synth.normal_f32(synth.generator(seed), (E,))
    z[17] = np.inf
    rows.append(z)
    rows.append(np.full(E, -np.inf, np.float32))
    lg = np.stack(rows)[:R].astype(np.float32)
    assert lg.shape == (R, E)
    return lg


def test_routing_ties_bit_exact(sv):
    """256 experts, top-8: the indices match the oracle's exactly on rows full
    of ties (across 64-lane slots and between -0 and +0) and on rows with
    infinities and NaNs; the weights match where finite and are NaN at the
    same places."""
    E, k, hidden, inter, R = 256, 8, 256, 256, 12
    (g, u, d), _ = _small_moe(E, hidden, inter, False, 150)
    lg = _tie_logits(R, E, 151)
    x = synth.normal_bf16(synth.generator(152), (R, hidden))
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, hidden, inter, E, k, dev(g), dev(u), dev(d))
    y = empty((R, hidden), "f32")
    ti = empty((R, k), "i32")
    tw = empty((R, k), "f32")
    say("vq2_moe_gemm routing ties E=256 k=8 R=12")
    sv.vq2_moe_gemm(desc, dev(x), dev(lg), y, ti, tw)
    gi, gw = host(ti), host(tw)
    widx, ww = oracle.route_topk(lg, k)
    assert np.array_equal(gi, widx), f"routing differs:\n{gi}\n{widx}"
    assert np.array_equal(np.isnan(gw), np.isnan(ww))
    fin = np.isfinite(ww)
    assert np.allclose(gw[fin], ww[fin], rtol=1e-5, atol=0)
    # the rows whose weights are all finite: the layer output against the oracle
    ok = [r for r in range(R) if np.all(np.isfinite(ww[r]))]
    want, _, _ = oracle.moe_layer(g, u, d, None, None, None, E, k, hidden, inter, x[ok], "bf16", lg[ok])
    assert_close(host(y)[ok], want, what="moe y (tie rows)")


@pytest.mark.parametrize("E,k", [(100, 8), (500, 16), (1024, 8)])
def test_routing_ties_wide_bit_exact(sv, E, k):
    """Router widths of 2, 8 and 16 logits per lane (the routing kernel's other
    instantiations): indices bit-exact with the oracle on integer-valued rows
    (ties across lanes and slots), a row with NaNs and -infs, and plain normal
    rows; weights close where finite.  The expert weights are zero blocks:
    only the routing outputs are compared."""
    hidden = inter = 256
    R = 6
    rng = np.random.default_rng(160 + E)
    rows = [rng.integers(-3, 4, size=E).astype(np.float32) for _ in range(3)]
    z = rng.integers(-2, 3, size=E).astype(np.float32)
    z[rng.choice(E, E // 3, replace=False)] = np.nan
    z[rng.choice(E, E // 3, replace=False)] = -np.inf
    rows.append(z)
    rows += [synth.normal_f32(synth.generator(161, E, i), (E,)) for i in range(2)]
    lg = np.stack(rows).astype(np.float32)
    nbytes = sv.sv_q2_matrix_bytes(inter, hidden) * E
    wz = empty((nbytes,), "u8").zero_()
    wd = empty((sv.sv_q2_matrix_bytes(hidden, inter) * E,), "u8").zero_()
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, hidden, inter, E, k, wz, wz, wd)
    x = synth.normal_bf16(synth.generator(162), (R, hidden))
    y = empty((R, hidden), "f32")
    ti = empty((R, k), "i32")
    tw = empty((R, k), "f32")
    say("vq2_moe_gemm routing", E, k, R)
    sv.vq2_moe_gemm(desc, dev(x), dev(lg), y, ti, tw)
    gi, gw = host(ti), host(tw)
    widx, ww = oracle.route_topk(lg, k)
    assert np.array_equal(gi, widx), f"routing differs:\n{gi}\n{widx}"
    assert np.array_equal(np.isnan(gw), np.isnan(ww))
    fin = np.isfinite(ww)
    assert np.allclose(gw[fin], ww[fin], rtol=1e-5, atol=0)


# ------------------------------------------------------------ lm head
@pytest.mark.parametrize("vocab,hidden,R,dt", [(1000, 1024, 5, "bf16"), (77, 256, 3, "f32"),
                                              (4096, 7168, 16, "bf16"), (33, 32, 40, "f32"),
                                              (1999, 1024, 1, "f32"), (3001, 2048, 4, "bf16"),
                                              (517, 3072, 2, "f32"), (700, 1024, 7, "bf16"),
                                              (300, 512, 64, "bf16"), (5000, 1024, 11, "bf16"),
                                              (2000, 2048, 7, "f32"), (70000, 512, 13, "bf16")])
def test_small_lm_head(sv, vocab, hidden, R, dt):
    p = synth.q8_random(synth.generator(107, vocab, hidden), vocab, hidden, 0.01)
    buf = p.packed()
    gen = synth.generator(108, R, hidden)
    h = synth.normal_bf16(gen, (R, hidden)) if dt == "bf16" else synth.normal_f32(gen, (R, hidden))
    out = empty((R, vocab), "f32")
    say("vq8_lmhead_gemm", vocab, hidden, R, dt)
    sv.vq8_lmhead_gemm(dev(buf), vocab, hidden, dev(h), out)
    want = oracle.lm_head_logits(buf, vocab, hidden, h, dt)
    assert_close(host(out), want, what=f"small head {vocab}x{hidden} R={R} {dt}")


# ------------------------------------------------------------- accept
def _run_accept(sv, S, K, V, target, tk, tp, draft, dk, tq, drafts, u):
    toks = empty((S, K + 1), "i32")
    nacc = empty((S,), "i32")
    say("spec_accept", S, K, V, tk, dk)
    sv.spec_accept(S, K, V, dev(target), tk, tp, dev(draft) if K else None, dk, tq,
                   dev(drafts) if K else None, dev(u), toks, nacc)
    return host(toks), host(nacc)


def test_tiny_accept_probs_bit_exact(sv):
    """Identical fp32 p, q and u: decisions and tokens must match exactly."""
    t = synth.tiny()
    p = np.stack([oracle.softmax_t(r, 1.0) for r in t.target_logits]).astype(np.float32)
    q = np.stack([oracle.softmax_t(r, 1.0) for r in t.draft_logits]).astype(np.float32)
    toks, nacc = _run_accept(sv, 1, 4, 32, p, PROBS, 1.0, q, PROBS, 1.0, t.drafts, t.uniforms)
    wt, wn = oracle.spec_accept(1, 4, 32, p, PROBS, 1.0, q, PROBS, 1.0, t.drafts, t.uniforms)
    assert np.array_equal(nacc, wn) and np.array_equal(toks, wt)


def test_tiny_accept_logits(sv):
    t = synth.tiny()
    toks, nacc = _run_accept(sv, 1, 4, 32, t.target_logits, LOGITS, 1.0, t.draft_logits, LOGITS,
                             1.0, t.drafts, t.uniforms)
    wt, wn = oracle.spec_accept(1, 4, 32, t.target_logits, LOGITS, 1.0, t.draft_logits, LOGITS,
                                1.0, t.drafts, t.uniforms)
    p_rows = [oracle.softmax_t(r, 1.0) for r in t.target_logits]
    q_rows = [oracle.softmax_t(r, 1.0) for r in t.draft_logits]
    if not accept_flags(p_rows, q_rows, t.drafts[0], t.uniforms[0], int(wn[0])):
        assert nacc[0] == wn[0]
        assert np.array_equal(toks, wt)


def test_accept_many_sequences_probs(sv):
    """Random p, q (zeros included) over many sequences: exact agreement."""
    rng = np.random.default_rng(9)
    S, K, V = 200, 5, 50
    def rows(n):
        w = rng.random((n, V)) * (rng.random((n, V)) > 0.3)
        w[:, 0] += 1e-3
        return (w / w.sum(1, keepdims=True)).astype(np.float32)
    p, q = rows(S * (K + 1)), rows(S * K)
    drafts = np.stack([[rng.choice(V, p=q[s * K + i] / q[s * K + i].sum()) for i in range(K)]
                       for s in range(S)]).astype(np.int32)
    u = synth.uniform24(synth.generator(110), S * (K + 1)).reshape(S, K + 1)
    toks, nacc = _run_accept(sv, S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u)
    wt, wn = oracle.spec_accept(S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u)
    assert np.array_equal(nacc, wn)
    bad = [s for s in range(S) if not np.array_equal(toks[s], wt[s])]
    # tokens may differ only where the sampling target sits on a CDF boundary
    for s in bad:
        n = wn[s]
        w = (np.maximum(p[s * (K + 1) + n].astype(np.float64) - q[s * K + n], 0) if n < K
             else p[s * (K + 1) + K].astype(np.float64))
        assert sample_flag(w, u[s, K]), s
    assert set(np.unique(wn).tolist()) > {0}      # the cases mix accepts and rejects


def test_accept_most_drafts_probs(sv):
    """K = 31 drafts (the limit) on probability rows, drafts drawn from q:
    agreement with the oracle, with chains that stop early, deep into the
    drafts, and after all 31 (q close to p)."""
    rng = np.random.default_rng(12)
    S, K, V = 6, 31, 40
    w = rng.random((S * (K + 1), V)) + 0.05
    p = (w / w.sum(1, keepdims=True)).astype(np.float32)
    qw = p[np.arange(S * (K + 1)).reshape(S, K + 1)[:, :K].reshape(-1)].astype(np.float64)
    qw = qw * (1.0 + 0.6 * rng.random(qw.shape))
    q = (qw / qw.sum(1, keepdims=True)).astype(np.float32)
    drafts = np.stack([[rng.choice(V, p=q[s * K + i] / q[s * K + i].sum()) for i in range(K)]
                       for s in range(S)]).astype(np.int32)
    u = synth.uniform24(synth.generator(111), S * (K + 1)).reshape(S, K + 1)
    toks, nacc = _run_accept(sv, S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u)
    wt, wn = oracle.spec_accept(S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u)
    assert np.array_equal(nacc, wn)
    for s in range(S):
        if not np.array_equal(toks[s], wt[s]):
            n = wn[s]
            wr = (np.maximum(p[s * (K + 1) + n].astype(np.float64) - q[s * K + n], 0) if n < K
                  else p[s * (K + 1) + K].astype(np.float64))
            assert sample_flag(wr, u[s, K]), s
    assert wn.max() == K and wn.min() < 8, wn   # chains stop early and run to the bonus


def _check_accept(S, K, V, target, tk, tp, draft, dk, tq, drafts, u, toks, nacc):
    """GPU outputs against the oracle's: invalid sequences all -1; decisions
    equal unless the oracle made one inside the flag band; tokens equal
    unless the sampling target sits on a CDF boundary."""
    wt, wn = oracle.spec_accept(S, K, V, target, tk, tp, draft, dk, tq, drafts, u)
    tg = np.asarray(target, np.float32).reshape(S, K + 1, V)
    dr = np.asarray(draft, np.float32).reshape(S, K, V) if K else None

    dist = oracle.distribution

    for s in range(S):
        if wn[s] < 0:
            assert nacc[s] == -1 and np.all(toks[s] == -1), f"sequence {s}: {nacc[s]} {toks[s]}"
            continue
        p_rows = [dist(tg[s, i], tk, tp) for i in range(K + 1)]
        q_rows = [dist(dr[s, i], dk, tq) for i in range(K)]
        if accept_flags(p_rows, q_rows, drafts[s], u[s], int(wn[s])):
            continue
        assert nacc[s] == wn[s], f"sequence {s}: n_accepted {nacc[s]} vs oracle {wn[s]}"
        if not np.array_equal(toks[s], wt[s]):
            n = int(wn[s])
            w = np.maximum(p_rows[n] - q_rows[n], 0.0) if n < K else p_rows[K]
            if not w.sum() > 0:
                w = p_rows[n]
            assert sample_flag(w, u[s, K]), f"sequence {s}: tokens {toks[s]} vs oracle {wt[s]}"
    return wn


def _logit_inputs(key, S, K, V, noise, T):
    g = synth.generator(key)
    z = synth.normal(g, S * (K + 1) * V, 2.0).astype(np.float32).reshape(S * (K + 1), V)
    zq = (z.reshape(S, K + 1, V)[:, :K].reshape(S * K, V).astype(np.float64)
          + synth.normal(g, S * K * V, noise).reshape(S * K, V)).astype(np.float32)
    drafts = synth.gumbel_drafts(zq, T, g).reshape(S, K)
    u = synth.uniform24(g, S * (K + 1)).reshape(S, K + 1)
    return z, zq, drafts, u


def test_accept_bonus_only(sv):
    """K = 0: one sample from p_0 per sequence (ragged last chunk)."""
    g = synth.generator(130)
    S, V = 3, 5000
    z = synth.normal(g, S * V, 2.0).astype(np.float32).reshape(S, V)
    u = synth.uniform24(g, S).reshape(S, 1)
    drafts = np.zeros((S, 0), np.int32)
    toks, nacc = _run_accept(sv, S, 0, V, z, LOGITS, 0.7, None, LOGITS, 0.7, drafts, u)
    wn = _check_accept(S, 0, V, z, LOGITS, 0.7, None, LOGITS, 0.7, drafts, u, toks, nacc)
    assert np.all(wn == 0)


def test_accept_one_token_vocabulary(sv):
    """V = 1, the degenerate vocabulary: p = q = 1 at the only token, so every
    draft is accepted and the bonus token is 0, under both rules and both
    kinds of rows."""
    S, K, V = 3, 4, 1
    z = synth.normal(synth.generator(131), S * (K + 1), 1.0).astype(np.float32).reshape(S * (K + 1), V)
    zq = synth.normal(synth.generator(132), S * K, 1.0).astype(np.float32).reshape(S * K, V)
    drafts = np.zeros((S, K), np.int32)
    u = synth.uniform24(synth.generator(133), S * (K + 1)).reshape(S, K + 1)
    for tk, t, q in ((LOGITS, 0.8, zq), (PROBS, 1.0, np.ones((S * K, V), np.float32))):
        tv = z if tk == LOGITS else np.ones((S * (K + 1), V), np.float32)
        toks, nacc = _run_accept(sv, S, K, V, tv, tk, t, q, tk, t, drafts, u)
        assert np.all(nacc == K) and np.all(toks == 0), (toks, nacc)
        wt, wn = oracle.spec_accept(S, K, V, tv, tk, t, q, tk, t, drafts, u)
        assert np.array_equal(wn, nacc) and np.array_equal(wt, toks)
        toks, nacc = _run_tsm(sv, S, K, V, tv, tk, t, drafts, u)
        assert np.all(nacc == K) and np.all(toks == 0), (toks, nacc)


def test_accept_invalid_sequences(sv):
    """A token outside [0, V), a uniform of 1, a NaN draft value and an
    infinite target value each void their own sequence only."""
    S, K, V = 5, 3, 4100
    z, zq, drafts, u = _logit_inputs(131, S, K, V, 1.0, 1.0)
    drafts[1, 2] = V
    u[2, 0] = 1.0
    zq[3 * K + 1, 77] = np.nan
    z[4 * (K + 1) + K, 5] = np.inf
    toks, nacc = _run_accept(sv, S, K, V, z, LOGITS, 1.0, zq, LOGITS, 1.0, drafts, u)
    wn = _check_accept(S, K, V, z, LOGITS, 1.0, zq, LOGITS, 1.0, drafts, u, toks, nacc)
    assert wn[0] >= 0 and np.all(wn[1:] == -1)


def test_accept_residual_vanished(sv):
    """q = p * (1 + 1e-5) as probabilities: a rejection leaves an all-zero
    residual, so the replacement is sampled from p itself."""
    g = synth.generator(132)
    S, K, V = 2, 2, 3000
    w = np.abs(synth.normal(g, S * (K + 1) * V, 1.0)).reshape(S * (K + 1), V) + 1e-3
    p = (w / w.sum(1, keepdims=True)).astype(np.float32)
    q = (p.reshape(S, K + 1, V)[:, :K].reshape(S * K, V) * np.float32(1.00001)).astype(np.float32)
    assert np.all(q > p.reshape(S, K + 1, V)[:, :K].reshape(S * K, V))
    drafts = np.array([[5, 9], [11, 13]], np.int32)
    u = np.array([[0.999995, 0.5, 0.3], [0.1, 0.2, 0.6]], np.float32)
    toks, nacc = _run_accept(sv, S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u)
    wn = _check_accept(S, K, V, p, PROBS, 1.0, q, PROBS, 1.0, drafts, u, toks, nacc)
    assert wn.tolist() == [0, 2]


def test_accept_largest_vocabulary(sv):
    """V = 524,288, the largest vocabulary the library takes (256 chunks)."""
    S, K, V = 2, 2, 256 * 2048
    z, zq, drafts, u = _logit_inputs(133, S, K, V, 1.5, 0.8)
    toks, nacc = _run_accept(sv, S, K, V, z, LOGITS, 0.8, zq, LOGITS, 0.8, drafts, u)
    _check_accept(S, K, V, z, LOGITS, 0.8, zq, LOGITS, 0.8, drafts, u, toks, nacc)


def _greedy_inputs(key, S, K, V):
    """Integer logits in [-50, 50): every row's maximum is tied at many
    positions spread over many chunks.  Drafts equal the target row's first
    maximum 3 times in 4, so every prefix length occurs."""
    rng = np.random.default_rng(key)
    z = rng.integers(-50, 50, size=(S * (K + 1), V)).astype(np.float32)
    zq = rng.integers(-50, 50, size=(S * K, V)).astype(np.float32)
    drafts = rng.integers(0, V, size=(S, K)).astype(np.int32)
    first = z.reshape(S, K + 1, V)[:, :K].argmax(-1)
    drafts = np.where(rng.random((S, K)) < 0.75, first, drafts).astype(np.int32)
    u = synth.uniform24(synth.generator(key), S * (K + 1)).reshape(S, K + 1)
    return z, zq, drafts, u


@pytest.mark.parametrize("t_q", [1.0, 0.0])
def test_accept_greedy_target(sv, t_q):
    """T_p = 0 (greedy): exact agreement with the oracle, and with the
    prefix-match form (drafts kept while they equal the target's first
    largest logit, then that row's first largest logit)."""
    S, K, V = 48, 4, 70000
    z, zq, drafts, u = _greedy_inputs(140, S, K, V)
    toks, nacc = _run_accept(sv, S, K, V, z, LOGITS, 0.0, zq, LOGITS, t_q, drafts, u)
    wt, wn = oracle.spec_accept(S, K, V, z, LOGITS, 0.0, zq, LOGITS, t_q, drafts, u)
    assert np.array_equal(nacc, wn) and np.array_equal(toks, wt)
    best = z.reshape(S, K + 1, V).argmax(-1)
    for s in range(S):
        n = 0
        while n < K and drafts[s, n] == best[s, n]:
            n += 1
        assert nacc[s] == n and toks[s, :n].tolist() == drafts[s, :n].tolist() and toks[s, n] == best[s, n]
    assert set(nacc.tolist()) == set(range(K + 1))


def test_accept_greedy_draft(sv):
    """T_q = 0 with a soft target (T_p = 0.8): q is one-hot at the draft
    row's first maximum and the drafts are those maxima."""
    S, K, V = 16, 3, 9000
    g = synth.generator(141)
    z = synth.normal(g, S * (K + 1) * V, 2.0).astype(np.float32).reshape(S * (K + 1), V)
    zq = (z.reshape(S, K + 1, V)[:, :K].reshape(S * K, V).astype(np.float64)
          + synth.normal(g, S * K * V, 0.3).reshape(S * K, V)).astype(np.float32)
    drafts = zq.argmax(-1).reshape(S, K).astype(np.int32)
    u = synth.uniform24(g, S * (K + 1)).reshape(S, K + 1)
    toks, nacc = _run_accept(sv, S, K, V, z, LOGITS, 0.8, zq, LOGITS, 0.0, drafts, u)
    wn = _check_accept(S, K, V, z, LOGITS, 0.8, zq, LOGITS, 0.0, drafts, u, toks, nacc)
    assert np.all(wn >= 0)


# ------------------------------------------------- target-sample matching
def _run_tsm(sv, S, K, V, target, tk, tp, drafts, u):
    toks = empty((S, K + 1), "i32")
    nacc = empty((S,), "i32")
    say("spec_accept_target_sample", S, K, V, tk, tp)
    sv.spec_accept_target_sample(S, K, V, dev(target), tk, tp, dev(drafts) if K else None, dev(u),
                                 toks, nacc)
    return host(toks), host(nacc)


def test_tsm_many_sequences_probs(sv):
    """Random probability rows (zeros included), drafts equal to the
    target's own sample 3 times in 4: agreement with the oracle, every prefix
    length present."""
    rng = np.random.default_rng(31)
    S, K, V = 200, 5, 50
    w = rng.random((S * (K + 1), V)) * (rng.random((S * (K + 1), V)) > 0.3)
    w[:, 0] += 1e-3
    p = (w / w.sum(1, keepdims=True)).astype(np.float32)
    u = synth.uniform24(synth.generator(150), S * (K + 1)).reshape(S, K + 1)
    drafts = matching_drafts(S, K, V, p, PROBS, 1.0, u, 0.75, rng)
    toks, nacc = _run_tsm(sv, S, K, V, p, PROBS, 1.0, drafts, u)
    wn, flagged = check_target_sample(S, K, V, p, PROBS, 1.0, drafts, u, toks, nacc)
    assert set(wn.tolist()) == set(range(K + 1)) and flagged <= 2


def test_tsm_most_drafts_probs(sv):
    """Target-sample matching with K = 31 drafts (the limit): agreement with
    the oracle, prefixes of many lengths."""
    rng = np.random.default_rng(32)
    S, K, V = 8, 31, 40
    w = rng.random((S * (K + 1), V)) * (rng.random((S * (K + 1), V)) > 0.2)
    w[:, 0] += 1e-3
    p = (w / w.sum(1, keepdims=True)).astype(np.float32)
    u = synth.uniform24(synth.generator(151), S * (K + 1)).reshape(S, K + 1)
    drafts = matching_drafts(S, K, V, p, PROBS, 1.0, u, 0.9, rng)
    toks, nacc = _run_tsm(sv, S, K, V, p, PROBS, 1.0, drafts, u)
    wn, flagged = check_target_sample(S, K, V, p, PROBS, 1.0, drafts, u, toks, nacc)
    assert flagged <= 1 and wn.max() >= 4, wn


def test_tsm_logits_ragged_and_invalid(sv):
    """Logit rows at T = 0.8 over V = 4,100 (three chunks, a ragged one); a
    token outside [0, V), a uniform of 1 and an infinite target value each
    void their own sequence only."""
    rng = np.random.default_rng(32)
    S, K, V = 7, 3, 4100
    z, _, _, u = _logit_inputs(151, S, K, V, 1.0, 0.8)
    drafts = matching_drafts(S, K, V, z, LOGITS, 0.8, u, 0.8, rng)
    drafts[1, 2] = V
    u[2, 0] = 1.0
    z[4 * (K + 1) + K, 5] = np.inf
    toks, nacc = _run_tsm(sv, S, K, V, z, LOGITS, 0.8, drafts, u)
    wn, _ = check_target_sample(S, K, V, z, LOGITS, 0.8, drafts, u, toks, nacc)
    assert wn[1] == -1 and wn[2] == -1 and wn[4] == -1 and np.all(wn[[0, 3, 5, 6]] >= 0)


def test_tsm_no_drafts_equals_bonus_sample(sv):
    """K = 0: the same token as spec_accept's bonus sample (both take the
    first entry whose running sum exceeds u Z; they sum in different chunk
    sizes, so only a u Z within rounding of a CDF boundary could differ)."""
    g = synth.generator(152)
    S, V = 6, 9000
    z = synth.normal(g, S * V, 2.0).astype(np.float32).reshape(S, V)
    u = synth.uniform24(g, S).reshape(S, 1)
    empty_d = np.zeros((S, 0), np.int32)
    a = _run_tsm(sv, S, 0, V, z, LOGITS, 0.7, empty_d, u)
    b = _run_accept(sv, S, 0, V, z, LOGITS, 0.7, None, LOGITS, 0.7, empty_d, u)
    assert np.array_equal(a[1], b[1])
    for s_ in range(S):
        if a[0][s_, 0] != b[0][s_, 0]:
            assert sample_flag(oracle.softmax_t(z[s_], 0.7), u[s_, 0]), s_
    check_target_sample(S, 0, V, z, LOGITS, 0.7, empty_d, u, *a)


def test_tsm_greedy_equals_pq_greedy(sv):
    """T_p = 0: target-sample matching and the p/q rule give the same output
    (the longest prefix of drafts equal to their rows' first maxima, then the
    next row's first maximum), exactly, at V = 70,000 with ties across chunks."""
    S, K, V = 48, 4, 70000
    z, zq, drafts, u = _greedy_inputs(153, S, K, V)
    a = _run_tsm(sv, S, K, V, z, LOGITS, 0.0, drafts, u)
    b = _run_accept(sv, S, K, V, z, LOGITS, 0.0, zq, LOGITS, 1.0, drafts, u)
    wt, wn = oracle.spec_accept_target_sample(S, K, V, z, LOGITS, 0.0, drafts, u)
    assert np.array_equal(a[0], wt) and np.array_equal(a[1], wn)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert set(wn.tolist()) == set(range(K + 1))


def test_tsm_largest_vocabulary(sv):
    """V = 524,288 (256 statistics chunks, 1,024 sampling chunks per row)."""
    rng = np.random.default_rng(34)
    S, K, V = 2, 2, 256 * 2048
    z, _, _, u = _logit_inputs(154, S, K, V, 1.5, 0.8)
    drafts = matching_drafts(S, K, V, z, LOGITS, 0.8, u, 0.9, rng)
    toks, nacc = _run_tsm(sv, S, K, V, z, LOGITS, 0.8, drafts, u)
    check_target_sample(S, K, V, z, LOGITS, 0.8, drafts, u, toks, nacc)


def _chi_square(counts, probs):
    n = counts.sum()
    e = n * probs
    keep = e > 0
    assert np.all(counts[~keep] == 0)
    return float(((counts[keep] - e[keep]) ** 2 / e[keep]).sum()), int(keep.sum()) - 1


def test_sampler_chi_square(sv):
    """The samplers' output distribution on the GPU: 16,384 sequences share
    one target row (V = 40, T = 1); the bonus tokens of spec_accept (K = 0)
    and the first emitted tokens of target-sample matching (K = 2, fixed
    drafts: lossless, so distributed as p_0 whatever the drafts) are binned
    and tested with chi-square against p_0 (threshold 96: the 1e-6 tail for
    39 degrees of freedom is 96.1); the acceptance of draft 0 must also match
    p_0(draft 0) within 5 standard deviations."""
    S, V = 16384, 40
    g = synth.generator(155)
    row = synth.normal(g, V, 1.5).astype(np.float32)
    p0 = oracle.softmax_t(row, 1.0)
    u1 = synth.uniform24(g, S).reshape(S, 1)
    toks, nacc = _run_accept(sv, S, 0, V, np.tile(row, (S, 1)), LOGITS, 1.0, None, LOGITS, 1.0,
                             np.zeros((S, 0), np.int32), u1)
    assert np.all(nacc == 0)
    chi, dof = _chi_square(np.bincount(toks[:, 0], minlength=V).astype(np.float64), p0)
    print(f"\n[chi2] spec_accept K=0: {chi:.1f} on {dof} dof")
    assert dof == V - 1 and chi < 96.0
    K = 2
    rows = np.tile(np.stack([row, row[::-1].copy(), row]), (S, 1)).astype(np.float32)
    d0 = int(np.argsort(p0)[-3])
    drafts = np.tile(np.array([[d0, 7]], np.int32), (S, 1))
    u3 = synth.uniform24(g, S * (K + 1)).reshape(S, K + 1)
    toks, nacc = _run_tsm(sv, S, K, V, rows, LOGITS, 1.0, drafts, u3)
    assert np.all(nacc >= 0)
    chi, dof = _chi_square(np.bincount(toks[:, 0], minlength=V).astype(np.float64), p0)
    acc = float((nacc >= 1).mean())
    sd = float(np.sqrt(p0[d0] * (1 - p0[d0]) / S))
    print(f"[chi2] target-sample matching, first token: {chi:.1f} on {dof} dof; "
          f"draft 0 accepted {acc:.4f} vs p0 {p0[d0]:.4f}")
    assert chi < 96.0 and abs(acc - p0[d0]) < 5 * sd
