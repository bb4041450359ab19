"""Pins of the oracle's block formats against hand-computed blocks, an
independent byte packer and exact rational arithmetic (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pack_q2_by_hand(q, sc, m, d, dm):
    """Byte image of a two-bit matrix from per-element fields, written from the
    layout definition: byte j of a block = q[4j] | q[4j+1]<<2 | q[4j+2]<<4 |
    q[4j+3]<<6; nibble byte = sc | m<<4; planes at 256-byte aligned offsets.
    q [nblk, 256], sc/m [nblk, 16], d/dm fp16 [nblk]."""
    nblk = q.shape[0]
    codes = bytearray()
    for b in range(nblk):
        for j in range(64):
            v = 0
            for t in range(4):
                v |= int(q[b, 4 * j + t]) << (2 * t)
            codes.append(v)
    nib = bytearray(int(sc[b, j]) | (int(m[b, j]) << 4) for b in range(nblk) for j in range(16))

    def pad(bs):
        return bytes(bs) + bytes((-len(bs)) % 256)

    return np.frombuffer(pad(codes) + pad(nib) + pad(np.asarray(d, np.float16).tobytes())
                         + pad(np.asarray(dm, np.float16).tobytes()), np.uint8)


def test_golden_blocks():
    cases = json.load(open(os.path.join(GOLDEN, "q2_blocks.json")))["cases"]
    for c in cases:
        q = np.full((1, 256), c["q"], np.uint8)
        sc = np.full((1, 16), c["sc"], np.uint8)
        m = np.full((1, 16), c["m"], np.uint8)
        d = np.array([float(Fraction(c["d"]))], np.float16)
        dm = np.array([float(Fraction(c["dmin"]))], np.float16)
        assert Fraction(float(d[0])) == Fraction(c["d"]), c["name"]       # fixture is fp16-exact
        assert Fraction(float(dm[0])) == Fraction(c["dmin"]), c["name"]
        buf = _pack_q2_by_hand(q, sc, m, d, dm)
        w = oracle.q2_dequant_f32(buf, 1, 256)
        assert w.dtype == np.float32 and w.shape == (1, 256)
        want = np.float32(float(Fraction(c["expect"])))
        assert Fraction(float(want)) == Fraction(c["expect"]), c["name"]
        assert np.all(w == want), (c["name"], w[0, :4], want)


def test_field_positions_brute_force():
    rng = np.random.default_rng(5)
    nblk = 3
    q = rng.integers(0, 4, size=(nblk, 256)).astype(np.uint8)
    sc = rng.integers(0, 16, size=(nblk, 16)).astype(np.uint8)
    m = rng.integers(0, 16, size=(nblk, 16)).astype(np.uint8)
    d = rng.normal(size=nblk).astype(np.float16)
    dm = rng.normal(size=nblk).astype(np.float16)
    buf = _pack_q2_by_hand(q, sc, m, d, dm)
    # one output row of 3 blocks (k_in = 768)
    gq, gsc, gm, du, dmu = oracle.q2_fields(buf, 1, 768)
    assert np.array_equal(gq.reshape(3, 256), q)
    assert np.array_equal(gsc.reshape(3, 16), sc)
    assert np.array_equal(gm.reshape(3, 16), m)
    # exact value of every element by Fraction arithmetic
    w = oracle.q2_dequant_f64(buf, 1, 768).reshape(3, 256)
    for b in range(nblk):
        for e in range(0, 256, 7):
            exact = Fraction(float(d[b])) * int(sc[b, e // 16]) * int(q[b, e]) \
                - Fraction(float(dm[b])) * int(m[b, e // 16])
            assert Fraction(float(w[b, e])) == exact


def test_rows_and_blocks_order():
    """Block b = n * nb + kb: output row n owns nb consecutive blocks."""
    n_out, k_in = 3, 512
    nb = 2
    q = np.zeros((n_out * nb, 256), np.uint8)
    sc = np.zeros((n_out * nb, 16), np.uint8)
    m = np.zeros((n_out * nb, 16), np.uint8)
    d = np.zeros(n_out * nb, np.float16)
    dm = np.zeros(n_out * nb, np.float16)
    for n in range(n_out):
        for kb in range(nb):
            b = n * nb + kb
            q[b] = 1
            sc[b] = 1
            d[b] = 10 * n + kb          # value identifies (n, kb)
    buf = _pack_q2_by_hand(q, sc, m, d, dm)
    w = oracle.q2_dequant_f32(buf, n_out, k_in)
    for n in range(n_out):
        assert np.all(w[n, :256] == 10 * n) and np.all(w[n, 256:] == 10 * n + 1)


def test_matrix_bytes():
    # at the workload shapes no padding occurs: 84 B per 256 weights, 34 B per 32
    assert oracle.q2_matrix_bytes(2048, 7168) == 84 * 2048 * 7168 // 256 == 4816896
    assert oracle.q2_matrix_bytes(7168, 2048) == 4816896
    assert oracle.q2_matrix_bytes(512, 256) == 84 * 512
    assert oracle.q8_matrix_bytes(129280, 7168) == 984596480
    # one block: every plane padded to 256 bytes
    assert oracle.q2_matrix_bytes(1, 256) == 4 * 256
    assert oracle.q8_matrix_bytes(1, 32) == 2 * 256


def test_generator_layout_agrees_with_oracle():
    """synth lays planes out; the oracle parses them independently."""
    p = synth.q2_random(synth.generator(9, 0), 8, 512, 0.02)
    buf = p.packed()
    assert buf.size == oracle.q2_matrix_bytes(8, 512)
    q, sc, m, du, dmu = oracle.q2_fields(buf, 8, 512)
    assert np.array_equal((sc | (m << 4)).reshape(-1), p.sc)
    assert np.array_equal(du.reshape(-1), (p.d.astype(np.float64) * 2 ** 24).astype(np.int64))
    p8 = synth.q8_random(synth.generator(9, 1), 4, 64, 0.01)
    b8 = p8.packed()
    assert b8.size == oracle.q8_matrix_bytes(4, 64)
    q8, d8 = oracle.q8_fields(b8, 4, 64)
    assert np.array_equal(q8.reshape(-1), p8.qs) and np.array_equal(d8.reshape(-1), p8.d)


def test_q8_hand_block():
    qs = np.zeros(64, np.int8)
    qs[0], qs[1], qs[31], qs[32] = -127, 127, 5, -1
    d = np.array([0.5, 0.125], np.float16)
    buf = synth.pack_planes(qs, d)
    w = oracle.q8_dequant_f32(buf, 1, 64)
    assert w[0, 0] == -63.5 and w[0, 1] == 63.5 and w[0, 31] == 2.5 and w[0, 32] == -0.125
    assert np.all(w[0, 2:31] == 0) and np.all(w[0, 33:] == 0)


def test_q2_dequant_rounds_once():
    """Random fields: the fp32 value is the exact rational rounded once."""
    p = synth.q2_random(synth.generator(11, 0), 4, 256, 0.02)
    buf = p.packed()
    w32 = oracle.q2_dequant_f32(buf, 4, 256)
    exact = oracle.q2_dequant_units(buf, 4, 256)
    for n in range(4):
        for e in range(0, 256, 5):
            fr = Fraction(int(exact[n, e]), 2 ** 24)
            got = Fraction(float(w32[n, e]))
            # got must be an fp32 neighbour of fr no farther than half a spacing
            spacing = Fraction(float(np.spacing(np.float32(abs(float(fr)) or 1e-30))))
            assert abs(got - fr) <= spacing / 2
