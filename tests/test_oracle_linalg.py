"""Pins of the oracle's products, SwiGLU, routing and MoE combine against
exact rationals, closed forms and brute force (CPU only)."""
import math
from fractions import Fraction

import numpy as np

import oracle
import synth


def _const_q2(n_out, k_in, d, dmin=0.0, sc=1, m=0, q=1):
    """A two-bit matrix whose every weight is d*sc*q - dmin*m."""
    nblk = n_out * k_in // 256
    byte = q | (q << 2) | (q << 4) | (q << 6)
    return synth.pack_planes(np.full(nblk * 64, byte, np.uint8),
                             np.full(nblk * 16, sc | (m << 4), np.uint8),
                             np.full(nblk, d, np.float16), np.full(nblk, dmin, np.float16))


def test_gemm_against_exact_rationals():
    n_out, k_in, R = 8, 256, 2
    p = synth.q2_random(synth.generator(21, 0), n_out, k_in, 0.02)
    buf = p.packed()
    x = synth.normal_f32(synth.generator(21, 1), (R, k_in))
    y = oracle.plain_layer(buf, n_out, k_in, x, "f32")
    units = oracle.q2_dequant_units(buf, n_out, k_in)
    for r in range(R):
        for n in range(n_out):
            exact = sum(Fraction(int(units[n, k]), 2 ** 24) * Fraction(float(x[r, k]))
                        for k in range(k_in))
            absum = sum(abs(Fraction(int(units[n, k]), 2 ** 24) * Fraction(float(x[r, k])))
                        for k in range(k_in))
            gamma = k_in * 2.0 ** -53 / (1 - k_in * 2.0 ** -53)
            assert abs(Fraction(float(y[r, n])) - exact) <= Fraction(gamma) * absum


def test_plain_layer_closed_form():
    """All weights equal c: every output is c * sum(x)."""
    c = 0.375
    buf = _const_q2(16, 512, c)
    x = synth.normal_f32(synth.generator(22, 1), (3, 512))
    y = oracle.plain_layer(buf, 16, 512, x, "f32")
    want = np.array([math.fsum(float(v) for v in x[r]) * c for r in range(3)])
    assert np.allclose(y, want[:, None], rtol=1e-13, atol=1e-12)
    # min term: d=0, dmin=0.5, m=3 -> every weight -1.5
    buf2 = _const_q2(16, 512, 0.0, dmin=0.5, sc=7, m=3, q=2)
    y2 = oracle.plain_layer(buf2, 16, 512, x, "f32")
    assert np.allclose(y2, -1.5 * want[:, None] / c, rtol=1e-13, atol=1e-12)


def test_bf16_rows_are_exact():
    bits = np.array([[0x3F80, 0xC000, 0x0001, 0x7F7F]], np.uint16)   # 1, -2, tiny denormal, max
    buf = _const_q2(1, 256, 1.0)
    x = np.zeros((1, 256), np.uint16)
    x[0, :4] = bits
    y = oracle.plain_layer(buf, 1, 256, x, "bf16")
    want = 1.0 - 2.0 + 2.0 ** -133 + float(np.float32(3.3895313892515355e38))
    assert y[0, 0] == want


def test_silu():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    big = np.array([40.0, 100.0])
    assert np.allclose(oracle.silu(big), big, rtol=1e-15)
    g = np.linspace(-30, 30, 61)
    sig = 1.0 / (1.0 + np.exp(-g))
    assert np.allclose(oracle.silu(g), g * sig, rtol=1e-14, atol=1e-300)
    # silu(-x) = silu(x) - x
    assert np.allclose(oracle.silu(-g), oracle.silu(g) - g, rtol=1e-12, atol=1e-12)
    far = oracle.silu(np.array([-800.0, -1e4]))
    assert np.all(np.isfinite(far)) and np.all(far <= 0) and np.all(far > -1e-300)


def test_route_topk_brute_force():
    rng = np.random.default_rng(3)
    E, k = 16, 4
    for trial in range(50):
        z = rng.integers(-3, 4, size=(5, E)).astype(np.float32)   # many ties
        idx, w = oracle.route_topk(z, k)
        for r in range(5):
            # repeated selection of the largest remaining, lowest index on ties
            left = list(range(E))
            want = []
            for _ in range(k):
                best = left[0]
                for e in left:
                    if z[r, e] > z[r, best]:
                        best = e
                want.append(best)
                left.remove(best)
            assert idx[r].tolist() == want
            denom = math.fsum(math.exp(float(v)) for v in z[r])
            assert np.allclose(w[r], [math.exp(float(z[r, e])) / denom for e in want], rtol=1e-14)


def test_moe_closed_form():
    """Constant experts: W_g = a_e, W_u = b_e, W_d = c_e everywhere, so
    FFN_e(x) = c_e * inter * silu(a_e S) * b_e S with S = sum(x), in every
    output element; the layer is the top-k softmax-weighted sum plus the
    shared expert."""
    hidden, inter, E, k, R = 256, 256, 6, 2, 3
    a = [0.25, -0.5, 0.125, 1.0, -0.25, 0.5, 0.0625]      # index E: shared
    b = [0.5, 0.25, -0.125, 0.0625, 1.0, -1.0, 0.25]
    c = [2.0 ** -6, -2.0 ** -5, 2.0 ** -4, 2.0 ** -7, -2.0 ** -6, 2.0 ** -8, 2.0 ** -5]
    gate = np.concatenate([_const_q2(inter, hidden, a[e]) for e in range(E)])
    up = np.concatenate([_const_q2(inter, hidden, b[e]) for e in range(E)])
    down = np.concatenate([_const_q2(hidden, inter, c[e]) for e in range(E)])
    sg, su, sd = _const_q2(inter, hidden, a[E]), _const_q2(inter, hidden, b[E]), _const_q2(hidden, inter, c[E])
    x = (synth.normal_f32(synth.generator(23, 0), (R, hidden)) * 0.05).astype(np.float32)
    logits = np.array([[0.1, 2.0, -1.0, 0.5, 0.5, 3.0],
                       [1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
                       [-2.0, 0.0, 4.0, -1.0, 2.5, 0.0]], np.float32)
    y, idx, w = oracle.moe_layer(gate, up, down, sg, su, sd, E, k, hidden, inter, x, "f32", logits)

    def ffn(e, S):
        g = a[e] * S
        return c[e] * inter * (g / (1 + math.exp(-g))) * b[e] * S

    want_idx = [[5, 1], [0, 1], [2, 4]]
    assert idx.tolist() == want_idx
    for r in range(R):
        S = math.fsum(float(v) for v in x[r])
        den = math.fsum(math.exp(float(v)) for v in logits[r])
        val = sum(math.exp(float(logits[r, e])) / den * ffn(e, S) for e in want_idx[r]) + ffn(E, S)
        assert np.allclose(y[r], val, rtol=1e-10, atol=1e-12)


def _const_q8(n_out, k_in, d, q):
    """An eight-bit matrix whose every weight is d*q."""
    nblk = n_out * k_in // 32
    return synth.pack_planes(np.full(nblk * 32, q, np.int8), np.full(nblk, d, np.float16))


def test_moe_eight_bit_shared_closed_form():
    """The shared expert in eight-bit blocks: constant matrices d*q, so
    FFN_shared(x) = c * inter * silu(a S) * b S with a, b, c the products
    d*q of gate, up and down; routed experts two-bit as before.  Also: the
    two formats give the same layer when they hold the same weights."""
    hidden, inter, E, k, R = 256, 256, 3, 1, 2
    gate = np.concatenate([_const_q2(inter, hidden, 0.25 * (e + 1)) for e in range(E)])
    up = np.concatenate([_const_q2(inter, hidden, -0.5 * (e + 1)) for e in range(E)])
    down = np.concatenate([_const_q2(hidden, inter, 2.0 ** -(6 + e)) for e in range(E)])
    a, b, c = 0.125 * 3, -0.0625 * 5, 2.0 ** -9 * 7
    sg, su, sd = _const_q8(inter, hidden, 0.125, 3), _const_q8(inter, hidden, -0.0625, 5), _const_q8(hidden, inter, 2.0 ** -9, 7)
    x = (synth.normal_f32(synth.generator(26, 0), (R, hidden)) * 0.05).astype(np.float32)
    logits = np.array([[0.0, 1.0, -1.0], [2.0, 0.5, 0.25]], np.float32)
    y, idx, w = oracle.moe_layer(gate, up, down, sg, su, sd, E, k, hidden, inter, x, "f32", logits,
                                 shared_format="q8")
    y0, _, _ = oracle.moe_layer(gate, up, down, None, None, None, E, k, hidden, inter, x, "f32", logits)
    assert idx.tolist() == [[1], [0]]
    for r in range(R):
        S = math.fsum(float(v) for v in x[r])
        g = a * S
        shared = c * inter * (g / (1 + math.exp(-g))) * b * S
        assert np.allclose(y[r] - y0[r], shared, rtol=1e-10, atol=1e-14)
    # the same constant weights as two-bit blocks (d*sc*q with sc = 1, q = 1)
    sg2, su2, sd2 = _const_q2(inter, hidden, a), _const_q2(inter, hidden, b), _const_q2(hidden, inter, c)
    y2, _, _ = oracle.moe_layer(gate, up, down, sg2, su2, sd2, E, k, hidden, inter, x, "f32", logits)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-15)


def test_moe_single_expert_no_router():
    hidden, inter = 256, 256
    g, u, d = _const_q2(inter, hidden, 0.5), _const_q2(inter, hidden, 0.25), _const_q2(hidden, inter, 2.0 ** -6)
    x = (synth.normal_f32(synth.generator(24, 0), (2, hidden)) * 0.1).astype(np.float32)
    y, idx, w = oracle.moe_layer(g, u, d, None, None, None, 1, 1, hidden, inter, x, "f32", None)
    for r in range(2):
        S = math.fsum(float(v) for v in x[r])
        gg = 0.5 * S
        assert np.allclose(y[r], 2.0 ** -6 * inter * gg / (1 + math.exp(-gg)) * 0.25 * S, rtol=1e-10)
    assert idx.tolist() == [[0], [0]] and np.all(w == 1.0)


def test_lm_head_against_exact_rationals():
    vocab, hidden, R = 7, 64, 2
    p = synth.q8_random(synth.generator(25, 0), vocab, hidden, 0.01)
    buf = p.packed()
    h = synth.normal_bf16(synth.generator(25, 1), (R, hidden))
    z = oracle.lm_head_logits(buf, vocab, hidden, h, "bf16", chunk=3)
    hx = synth.bf16_bits_to_f32(h)
    for r in range(R):
        for v in range(vocab):
            exact = sum(Fraction(float(p.d[(v * hidden + k) // 32])) * int(p.qs[v * hidden + k])
                        * Fraction(float(hx[r, k])) for k in range(hidden))
            assert abs(Fraction(float(z[r, v])) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)
    # a row sample returns the same columns
    zs = oracle.lm_head_logits(buf, vocab, hidden, h, "bf16", rows=[6, 0, 3])
    assert np.array_equal(zs, z[:, [6, 0, 3]])
