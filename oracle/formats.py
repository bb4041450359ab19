"""Block formats of the verifier weights, dequantised exactly (oracle; test
infrastructure only).

Sources: the *ds4-on-spark* README, introduction (model bullet), names a
two-bit "Q2_K" format for routed-expert weights and an eight-bit "Q8_0" format
for the output head; the pages give no bit layout.  The layout used here is the
reading fixed for this library:

Two-bit matrix [n_out x k_in], k_in % 256 == 0, nb = k_in / 256 blocks per
output row, block index b = n * nb + kb.  Four planes, each at a 256-byte
aligned offset from the start of the buffer:

  codes   nblk*64 bytes   element e of block b = (codes[64b + e//4] >> 2*(e%4)) & 3
  nibbles nblk*16 bytes   byte j (sub-block j, elements 16j..16j+15):
                          low nibble = scale sc, high nibble = min m
  d       nblk fp16       block scale
  dmin    nblk fp16       block min-scale

  w = d * sc * q - dmin * m      (the exact real value)

Eight-bit matrix: nb = k_in / 32, planes codes nblk*32 int8 and d nblk fp16;
w = d * q.

The "dequantised weight" of the two-bit format is the exact value rounded once
to fp32 (nearest, ties to even).  Every fp16 number is an integer multiple of
2^-24 below 2^40 in those units, so ``w * 2^24`` is an integer of at most 47
bits: it is formed here in int64, converted exactly to fp64 and rounded once to
fp32.  The eight-bit product d * q needs at most 18 significant bits and is
exact in fp32.
"""
from __future__ import annotations

import numpy as np


def _up256(n: int) -> int:
    return -(-n // 256) * 256


def q2_matrix_bytes(n_out: int, k_in: int) -> int:
    nblk = n_out * (k_in // 256)
    return _up256(nblk * 64) + _up256(nblk * 16) + 2 * _up256(nblk * 2)


def q8_matrix_bytes(n_out: int, k_in: int) -> int:
    nblk = n_out * (k_in // 32)
    return _up256(nblk * 32) + _up256(nblk * 2)


def q2_fields(buf: np.ndarray, n_out: int, k_in: int, rows=None):
    """Split a two-bit matrix buffer into per-element fields.

    Returns (q, sc, m, d_units, dm_units) for the selected output rows:
      q        uint8 [r, k_in]          codes 0..3
      sc, m    uint8 [r, k_in // 16]    nibbles per 16-element sub-block
      d_units  int64 [r, k_in // 256]   d in units of 2^-24
      dm_units int64 [r, k_in // 256]
    """
    assert k_in % 256 == 0
    buf = np.asarray(buf, np.uint8).reshape(-1)
    nb = k_in // 256
    nblk = n_out * nb
    o_codes = 0
    o_nib = o_codes + _up256(nblk * 64)
    o_d = o_nib + _up256(nblk * 16)
    o_dm = o_d + _up256(nblk * 2)
    assert buf.size >= o_dm + nblk * 2, "buffer too small for the matrix"
    codes = buf[o_codes:o_codes + nblk * 64].reshape(n_out, nb, 64)
    nib = buf[o_nib:o_nib + nblk * 16].reshape(n_out, nb, 16)
    d = buf[o_d:o_d + nblk * 2].view(np.float16).reshape(n_out, nb)
    dm = buf[o_dm:o_dm + nblk * 2].view(np.float16).reshape(n_out, nb)
    if rows is not None:
        codes, nib, d, dm = codes[rows], nib[rows], d[rows], dm[rows]
    r = codes.shape[0]
    # byte j of a block holds elements 4j .. 4j+3, element 4j+t in bits 2t, 2t+1
    q = np.empty((r, nb, 64, 4), np.uint8)
    for t in range(4):
        q[..., t] = (codes >> np.uint8(2 * t)) & np.uint8(3)
    q = q.reshape(r, k_in)
    sc = (nib & np.uint8(15)).reshape(r, nb * 16)
    m = (nib >> np.uint8(4)).reshape(r, nb * 16)
    d_units = (d.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    dm_units = (dm.astype(np.float64) * 2.0 ** 24).astype(np.int64)
    return q, sc, m, d_units, dm_units


def q2_dequant_units(buf, n_out: int, k_in: int, rows=None) -> np.ndarray:
    """Exact dequantised weights as int64 multiples of 2^-24, [r, k_in]."""
    q, sc, m, du, dmu = q2_fields(buf, n_out, k_in, rows)
    sc_e = np.repeat(sc, 16, axis=1).astype(np.int64)   # sub-block of element e is e // 16
    m_e = np.repeat(m, 16, axis=1).astype(np.int64)
    du_e = np.repeat(du, 256, axis=1)
    dmu_e = np.repeat(dmu, 256, axis=1)
    return du_e * sc_e * q.astype(np.int64) - dmu_e * m_e


def q2_dequant_f64(buf, n_out: int, k_in: int, rows=None) -> np.ndarray:
    """Exact real weights (|w * 2^24| < 2^47 fits fp64 exactly)."""
    return q2_dequant_units(buf, n_out, k_in, rows).astype(np.float64) * 2.0 ** -24


def q2_dequant_f32(buf, n_out: int, k_in: int, rows=None) -> np.ndarray:
    """Exact weights rounded once to fp32 (nearest, ties to even)."""
    u = q2_dequant_units(buf, n_out, k_in, rows).astype(np.float64)   # exact
    return u.astype(np.float32) * np.float32(2.0 ** -24)              # one rounding, exact scaling


def q8_fields(buf: np.ndarray, n_out: int, k_in: int, rows=None):
    """(q int8 [r, k_in], d fp16 [r, k_in // 32]) of an eight-bit matrix."""
    assert k_in % 32 == 0
    buf = np.asarray(buf, np.uint8).reshape(-1)
    nb = k_in // 32
    nblk = n_out * nb
    o_d = _up256(nblk * 32)
    assert buf.size >= o_d + nblk * 2, "buffer too small for the matrix"
    q = buf[:nblk * 32].view(np.int8).reshape(n_out, nb * 32)
    d = buf[o_d:o_d + nblk * 2].view(np.float16).reshape(n_out, nb)
    if rows is not None:
        q, d = q[rows], d[rows]
    return q, d


def q8_dequant_f64(buf, n_out: int, k_in: int, rows=None) -> np.ndarray:
    q, d = q8_fields(buf, n_out, k_in, rows)
    return q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)


def q8_dequant_f32(buf, n_out: int, k_in: int, rows=None) -> np.ndarray:
    """d * q is exact in fp32 (11-bit times 7-bit significands)."""
    return q8_dequant_f64(buf, n_out, k_in, rows).astype(np.float32)
