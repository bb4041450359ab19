"""Seeded synthetic inputs for the speculative-decoding verifier step.

Both sides of every parity check draw their inputs from here: the HIP
library (through its Python binding) and the CPU oracle.  The module
therefore holds *no arithmetic of the verifier itself* -- no dequantisation,
no matrix products, no softmax, no accept/reject rule.  It only draws random
numbers and lays them out:

* raw 64-bit words from a counter-free PCG64 stream, one stream per
  (config, purpose, ...) key built with ``numpy.random.SeedSequence``;
* uniforms on the 2^-24 grid, ``(raw >> 40) * 2^-24`` (exact in fp32);
* normals by Box-Muller (1958) on 53-bit uniforms in (0, 1], in fp64,
  then rounded once (round-to-nearest-even) to the storage dtype;
* bf16 rounding done with integer operations on the fp32 bit pattern;
* random code/scale bytes for the two-bit and eight-bit block formats, and
  the byte layout of their storage planes (each plane at a 256-byte-aligned
  offset).

The draft tokens of the drafter -- which the verifier receives as inputs --
are drawn here too, by the Gumbel-max device: the index of the maximum of
``z / T + G`` with ``G = -log(-log U)`` is a sample of ``softmax(z / T)``.
That is the drafter's job, not the verifier's, and the verifier never sees
how the tokens were drawn.

The workloads follow the five configurations of the verifier step:
``tiny`` (one dense two-bit layer plus a 32-token accept), ``expert`` (one
SwiGLU expert), ``moe_layer`` (256 routed experts + 1 shared, top-8),
``lm_head`` (a 129,280 x 7,168 eight-bit vocabulary head) and ``cohort``
(three sequences of five verifier rows).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

# ---------------------------------------------------------------- streams
CFG_TINY, CFG_EXPERT, CFG_MOE, CFG_LMHEAD, CFG_COHORT = 0, 1, 2, 3, 4

S_WEIGHTS, S_ACT, S_ROUTER, S_NOISE, S_DRAFTS, S_UNIFORMS, S_TARGET, S_HIDDEN = range(8)

# matrix ids inside one expert
M_GATE, M_UP, M_DOWN = 0, 1, 2

HIDDEN = 7168
INTER = 2048
N_ROUTED = 256
TOP_K = 8
VOCAB = 129280


def generator(*key: int) -> np.random.Generator:
    """PCG64 stream for one purpose; ``key`` is (config, stream, ...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def raw64(gen: np.random.Generator, n: int) -> np.ndarray:
    return gen.bit_generator.random_raw(int(n))


def uniform24(gen: np.random.Generator, n: int) -> np.ndarray:
    """fp32 uniforms in [0, 1) on the 2^-24 grid (exactly representable)."""
    r = raw64(gen, n) >> np.uint64(40)
    return (r.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def _uniform53_open(gen: np.random.Generator, n: int) -> np.ndarray:
    """fp64 uniforms in (0, 1] on the 2^-53 grid."""
    r = (raw64(gen, n) >> np.uint64(11)) + np.uint64(1)
    return r.astype(np.float64) * 2.0 ** -53


def normal(gen: np.random.Generator, n: int, sigma: float = 1.0) -> np.ndarray:
    """fp64 N(0, sigma^2) draws by the Box-Muller transform."""
    n = int(n)
    m = (n + 1) // 2
    u = _uniform53_open(gen, 2 * m)
    rad = np.sqrt(-2.0 * np.log(u[:m]))
    ang = (2.0 * np.pi) * u[m:]
    z = np.empty(2 * m, np.float64)
    z[0::2] = rad * np.cos(ang)
    z[1::2] = rad * np.sin(ang)
    return z[:n] * sigma


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) with integer operations."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(gen: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma^2) draws."""
    n = int(np.prod(shape))
    return f32_to_bf16_bits(normal(gen, n, sigma).astype(np.float32)).reshape(shape)


def normal_f32(gen: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    return normal(gen, n, sigma).astype(np.float32).reshape(shape)


# ------------------------------------------------------- block storage
def _align256(n: int) -> int:
    return (n + 255) // 256 * 256


def q2_plane_sizes(n_out: int, k_in: int):
    """Byte sizes of the four planes of a two-bit matrix: codes, scale/min
    nibbles, fp16 block scale, fp16 block min-scale."""
    nblk = n_out * (k_in // 256)
    return nblk * 64, nblk * 16, nblk * 2, nblk * 2


def q8_plane_sizes(n_out: int, k_in: int):
    nblk = n_out * (k_in // 32)
    return nblk * 32, nblk * 2


def pack_planes(*planes: np.ndarray) -> np.ndarray:
    """Concatenate byte planes, each starting at a 256-byte-aligned offset."""
    sizes = [p.nbytes for p in planes]
    total = sum(_align256(s) for s in sizes)
    out = np.zeros(total, np.uint8)
    off = 0
    for p, s in zip(planes, sizes):
        out[off:off + s] = np.ascontiguousarray(p).view(np.uint8).reshape(-1)
        off += _align256(s)
    return out


@dataclass
class Q2Planes:
    n_out: int
    k_in: int
    qs: np.ndarray   # uint8 [nblk*64]   four 2-bit codes per byte
    sc: np.ndarray   # uint8 [nblk*16]   low nibble scale, high nibble min
    d: np.ndarray    # float16 [nblk]
    dm: np.ndarray   # float16 [nblk]

    def packed(self) -> np.ndarray:
        return pack_planes(self.qs, self.sc, self.d, self.dm)


@dataclass
class Q8Planes:
    n_out: int
    k_in: int
    qs: np.ndarray   # int8 [nblk*32]
    d: np.ndarray    # float16 [nblk]

    def packed(self) -> np.ndarray:
        return pack_planes(self.qs, self.d)


def q2_random(gen: np.random.Generator, n_out: int, k_in: int, sigma: float) -> Q2Planes:
    """Uniform random code and nibble bytes; d, dmin ~ fp16(N(0, sigma^2))."""
    assert k_in % 256 == 0
    nq, ns, _, _ = q2_plane_sizes(n_out, k_in)
    nblk = nq // 64
    qs = gen.integers(0, 256, size=nq, dtype=np.uint8)
    sc = gen.integers(0, 256, size=ns, dtype=np.uint8)
    d = normal(gen, nblk, sigma).astype(np.float16)
    dm = normal(gen, nblk, sigma).astype(np.float16)
    return Q2Planes(n_out, k_in, qs, sc, d, dm)


def q8_random(gen: np.random.Generator, n_out: int, k_in: int, sigma: float) -> Q8Planes:
    """int8 codes uniform on -127..127; d ~ fp16(|N(0, sigma^2)|)."""
    assert k_in % 32 == 0
    nq, _ = q8_plane_sizes(n_out, k_in)
    qs = gen.integers(-127, 128, size=nq, dtype=np.int8)
    d = np.abs(normal(gen, nq // 32, sigma)).astype(np.float16)
    return Q8Planes(n_out, k_in, qs, d)


def gumbel_drafts(draft_logits: np.ndarray, temperature: float, gen: np.random.Generator) -> np.ndarray:
    """One drafter sample per row of ``draft_logits`` (Gumbel-max)."""
    z = np.asarray(draft_logits, np.float64)
    u = _uniform53_open(gen, z.size).reshape(z.shape)
    u = np.minimum(u, 1.0 - 2.0 ** -53)          # keep -log(u) > 0
    g = -np.log(-np.log(u))
    return np.argmax(z / float(temperature) + g, axis=-1).astype(np.int32)


# ------------------------------------------------------------ workloads
@dataclass
class Tiny:
    """One dense two-bit layer K=256 x N=512, R=4 fp32 rows, then an accept
    over a 32-token vocabulary with 4 drafts."""
    w: Q2Planes
    x: np.ndarray                 # float32 [4, 256]
    target_logits: np.ndarray     # float32 [5, 32]   (K+1 rows)
    draft_logits: np.ndarray      # float32 [4, 32]
    drafts: np.ndarray            # int32 [1, 4]
    uniforms: np.ndarray          # float32 [1, 5]
    temperature: float = 1.0


def tiny() -> Tiny:
    c = CFG_TINY
    w = q2_random(generator(c, S_WEIGHTS), 512, 256, 0.02)
    x = normal_f32(generator(c, S_ACT), (4, 256))
    tl = normal_f32(generator(c, S_TARGET), (5, 32), 2.0)
    noise = normal(generator(c, S_NOISE), 4 * 32).reshape(4, 32)
    dl = (tl[:4].astype(np.float64) + noise).astype(np.float32)
    drafts = gumbel_drafts(dl, 1.0, generator(c, S_DRAFTS)).reshape(1, 4)
    u = uniform24(generator(c, S_UNIFORMS), 5).reshape(1, 5)
    return Tiny(w, x, tl, dl, drafts, u, 1.0)


def expert_matrices(config_id: int, expert: int, sigma: float = 0.02,
                    hidden: int = HIDDEN, inter: int = INTER) -> Dict[int, Q2Planes]:
    """Gate [inter x hidden], up [inter x hidden], down [hidden x inter]."""
    out = {}
    for m, (n, k) in ((M_GATE, (inter, hidden)), (M_UP, (inter, hidden)), (M_DOWN, (hidden, inter))):
        out[m] = q2_random(generator(config_id, S_WEIGHTS, expert, m), n, k, sigma)
    return out


@dataclass
class Expert:
    """One SwiGLU expert in two-bit blocks with R bf16 rows."""
    mats: Dict[int, Q2Planes]
    x_bf16: np.ndarray            # uint16 [R, 7168]


def expert(R: int) -> Expert:
    assert 1 <= R <= 8
    mats = expert_matrices(CFG_EXPERT, 0)
    x = normal_bf16(generator(CFG_EXPERT, S_ACT), (8, HIDDEN))[:R].copy()
    return Expert(mats, x)


@dataclass
class MoeWeights:
    """256 routed experts + 1 shared, expert-major packed buffers."""
    gate: np.ndarray   # uint8 [256 * q2 bytes]
    up: np.ndarray
    down: np.ndarray
    s_gate: np.ndarray
    s_up: np.ndarray
    s_down: np.ndarray
    config_id: int = CFG_MOE

    def expert(self, e: int) -> Dict[int, Q2Planes]:
        return expert_matrices(self.config_id, e)


def moe_weights(config_id: int = CFG_MOE, n_routed: int = N_ROUTED) -> MoeWeights:
    bufs = {M_GATE: [], M_UP: [], M_DOWN: []}
    shared = None
    for e in range(n_routed + 1):
        mats = expert_matrices(config_id, e)
        packed = {m: mats[m].packed() for m in mats}
        if e == n_routed:
            shared = packed
        else:
            for m in packed:
                bufs[m].append(packed[m])
    return MoeWeights(np.concatenate(bufs[M_GATE]), np.concatenate(bufs[M_UP]),
                      np.concatenate(bufs[M_DOWN]), shared[M_GATE], shared[M_UP],
                      shared[M_DOWN], config_id)


@dataclass
class MoeRows:
    router_logits: np.ndarray    # float32 [R, 256]
    x_bf16: np.ndarray           # uint16 [R, 7168]


def moe_rows(R: int, config_id: int = CFG_MOE, sub: int = 0) -> MoeRows:
    lg = normal_f32(generator(config_id, S_ROUTER, sub), (R, N_ROUTED))
    x = normal_bf16(generator(config_id, S_ACT, sub), (R, HIDDEN))
    return MoeRows(lg, x)


def router_weights(config_id: int = CFG_MOE, n_experts: int = N_ROUTED, hidden: int = HIDDEN) -> Q8Planes:
    """Eight-bit router matrix [n_experts x hidden] (the router GEMV ahead of
    the top-k): the vocabulary head's format, scales ~ fp16(|N(0, 3e-4^2)|) so
    that the logits of unit-variance rows spread by about 2."""
    return q8_random(generator(config_id, S_ROUTER, 1 << 20), n_experts, hidden, 3e-4)


def shared_q8_weights(config_id: int = CFG_MOE, hidden: int = HIDDEN, inter: int = INTER,
                      sigma: float = 2e-3):
    """An eight-bit shared expert: gate, up [inter x hidden] and down
    [hidden x inter] in the vocabulary head's format, codes uniform on
    -127..127 and scales ~ fp16(|N(0, sigma^2)|), so that the weights spread
    about as much as the two-bit experts' (rms ~ 0.15)."""
    g = generator(config_id, S_WEIGHTS, 1 << 21)
    return (q8_random(g, inter, hidden, sigma), q8_random(g, inter, hidden, sigma),
            q8_random(g, hidden, inter, sigma))


def lm_head_weights(config_id: int = CFG_LMHEAD, vocab: int = VOCAB, hidden: int = HIDDEN) -> Q8Planes:
    return q8_random(generator(config_id, S_WEIGHTS), vocab, hidden, 0.01)


def lm_head_hidden(R: int, config_id: int = CFG_LMHEAD, sub: int = 0) -> np.ndarray:
    return normal_bf16(generator(config_id, S_HIDDEN, sub), (R, HIDDEN))


@dataclass
class AcceptInputs:
    """Draft side of one verifier cohort: S sequences of K drafts."""
    draft_logits: np.ndarray     # float32 [S*K, V]
    drafts: np.ndarray           # int32 [S, K]
    uniforms: np.ndarray         # float32 [S, K+1]


def accept_inputs(target_logits: np.ndarray, S: int, K: int, noise_sigma: float,
                  temperature_q: float, config_id: int, sub: int = 0) -> AcceptInputs:
    """Draft logits = target logits of each sequence's first K rows plus
    N(0, noise_sigma^2) noise; drafts drawn from softmax(draft / T_q);
    K+1 uniforms per sequence.  Each sequence has its own streams."""
    V = target_logits.shape[1]
    tl = np.asarray(target_logits, np.float32).reshape(S, K + 1, V)
    dl = np.empty((S, K, V), np.float32)
    drafts = np.empty((S, K), np.int32)
    u = np.empty((S, K + 1), np.float32)
    for s in range(S):
        noise = normal(generator(config_id, S_NOISE, sub, s), K * V, noise_sigma).reshape(K, V)
        dl[s] = (tl[s, :K].astype(np.float64) + noise).astype(np.float32)
        if K:
            drafts[s] = gumbel_drafts(dl[s], temperature_q, generator(config_id, S_DRAFTS, sub, s))
        u[s] = uniform24(generator(config_id, S_UNIFORMS, sub, s), K + 1)
    return AcceptInputs(dl.reshape(S * K, V), drafts, u)
