"""Products, SwiGLU experts, routing and the vocabulary head in fp64 (oracle;
test infrastructure only).

Each function is the plain definition of its step, with no blocking or fusion:

* ``gemm``           y[r, n] = sum_k W[n, k] x[r, k]  (one library matmul);
* ``silu``           silu(g) = g / (1 + e^-g);
* ``swiglu_expert``  W_d (silu(W_g x) * (W_u x)) -- the fused gate+up+SwiGLU expert
                     of the MoE decode path (*1x Spark tuned DSpark for
                     DeepSeek-V4-Flash* thread, Q&A answer 3);
* ``route_topk``     the k experts with the largest router logits (ties: lower
                     index first), weighted by the softmax probability over
                     all experts, not renormalised;
* ``moe_layer``      y_r = sum_s w[r, s] * FFN_e(r,s)(x_r) + FFN_shared(x_r): each
                     row goes to its top-k routed experts plus the always-on
                     shared expert (*ds4-on-spark* README, "Roofline" section:
                     a few of 256 routed experts per token plus the shared
                     expert);
* ``lm_head_logits`` logits = W h over the vocabulary, in row chunks.

Inputs are taken at their exact values (bf16 bit patterns are widened
exactly); every intermediate is fp64 and nothing is rounded to a narrower type.
"""
from __future__ import annotations

import numpy as np

from .formats import q2_dequant_f64, q8_dequant_f64, q2_matrix_bytes


def _exact_rows(x, dtype: str) -> np.ndarray:
    """Rows as fp64: ``dtype`` 'f32' (float32 values) or 'bf16' (uint16 bits)."""
    if dtype == "bf16":
        b = np.ascontiguousarray(x, np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32).astype(np.float64)
    return np.asarray(x, np.float32).astype(np.float64)


def gemm(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = x W^T for W [n, k] and rows x [r, k], fp64."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, np.float64)
    out = np.empty_like(g)
    lo = g < -700.0
    out[~lo] = g[~lo] / (1.0 + np.exp(-g[~lo]))
    e = np.exp(g[lo])
    out[lo] = g[lo] * e / (1.0 + e)
    return out


def swiglu_expert(w_gate, w_up, w_down, hidden: int, inter: int, x64: np.ndarray,
                  fmt: str = "q2") -> np.ndarray:
    """One SwiGLU expert on fp64 rows x64 [r, hidden] -> [r, hidden]; its
    matrices two-bit (fmt "q2") or eight-bit ("q8")."""
    deq = {"q2": q2_dequant_f64, "q8": q8_dequant_f64}[fmt]
    g = gemm(deq(w_gate, inter, hidden), x64)
    u = gemm(deq(w_up, inter, hidden), x64)
    h = silu(g) * u
    return gemm(deq(w_down, hidden, inter), h)


def route_topk(logits: np.ndarray, k: int):
    """(idx int32 [R, k], w fp64 [R, k]) from router logits [R, E]."""
    logits = np.asarray(logits, np.float32)
    R, E = logits.shape
    idx = np.empty((R, k), np.int32)
    w = np.empty((R, k), np.float64)
    for r in range(R):
        z = logits[r].astype(np.float64)
        order = np.lexsort((np.arange(E), -z))[:k]      # largest logit first, then lower index
        p = np.exp(z - z.max())
        p /= p.sum()
        idx[r] = order
        w[r] = p[order]
    return idx, w


def _slice_expert(buf, e: int, nbytes: int):
    return np.asarray(buf, np.uint8).reshape(-1)[e * nbytes:(e + 1) * nbytes]


def moe_layer(w_gate, w_up, w_down, s_gate, s_up, s_down, n_experts: int, top_k: int,
              hidden: int, inter: int, x, x_dtype: str, router_logits, shared_format: str = "q2"):
    """Routed + shared SwiGLU MoE layer.

    w_* hold ``n_experts`` expert-major two-bit matrices; s_* the shared
    expert (or None), two-bit or, with shared_format "q8", eight-bit (the
    format the pages' model keeps it in: *ds4-on-spark* README, introduction,
    the quantisation recipe).
    Returns (y fp64 [R, hidden], topk_idx int32 [R, k], topk_w fp64 [R, k]).
    """
    x64 = _exact_rows(x, x_dtype)
    R = x64.shape[0]
    if n_experts == 1 and router_logits is None:
        idx = np.zeros((R, top_k), np.int32)
        wts = np.ones((R, top_k), np.float64)
    else:
        idx, wts = route_topk(router_logits, top_k)
    bg = q2_matrix_bytes(inter, hidden)
    bd = q2_matrix_bytes(hidden, inter)
    y = np.zeros((R, hidden), np.float64)
    for e in sorted(set(idx.reshape(-1).tolist())):
        rows = sorted(set(np.nonzero(idx == e)[0].tolist()))
        ye = swiglu_expert(_slice_expert(w_gate, e, bg), _slice_expert(w_up, e, bg),
                           _slice_expert(w_down, e, bd), hidden, inter, x64[rows])
        for j, r in enumerate(rows):
            for s in np.nonzero(idx[r] == e)[0]:
                y[r] += wts[r, s] * ye[j]
    if s_gate is not None:
        y += swiglu_expert(s_gate, s_up, s_down, hidden, inter, x64, shared_format)
    return y, idx, wts


def plain_layer(w, n_out: int, k_in: int, x, x_dtype: str) -> np.ndarray:
    """y = W x for one two-bit matrix, fp64 [R, n_out]."""
    return gemm(q2_dequant_f64(w, n_out, k_in), _exact_rows(x, x_dtype))


def lm_head_logits(w, vocab: int, hidden: int, h, h_dtype: str, rows=None,
                   chunk: int = 8192) -> np.ndarray:
    """Vocabulary logits W h in fp64: [R, vocab], or [R, len(rows)] for a row sample."""
    h64 = _exact_rows(h, h_dtype)
    sel = np.arange(vocab) if rows is None else np.asarray(rows)
    out = np.empty((h64.shape[0], sel.size), np.float64)
    for c0 in range(0, sel.size, chunk):
        part = sel[c0:c0 + chunk]
        out[:, c0:c0 + part.size] = gemm(q8_dequant_f64(w, vocab, hidden, part), h64)
    return out
