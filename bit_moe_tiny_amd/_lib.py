"""ctypes binding of libspecverify (argument marshalling only).

Every function here forwards to the C ABI declared in ``include/specverify.h``
with the same name; all computation happens in the HIP kernels.  Tensors are
PyTorch device tensors (PyTorch provides device memory and streams); their
pointers and the current HIP stream are passed through unchanged.  There is no
fallback: if the shared library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_EINVAL, SV_EUNSUPPORTED, SV_EWORKSPACE, SV_EHIP, SV_ESCRATCH = range(6)
ACCEPT_SCRATCH_BYTES = 16 << 20   # SV_ACCEPT_SCRATCH_BYTES of the header
SV_F32, SV_BF16 = 0, 1
SV_FFN_PLAIN, SV_FFN_SWIGLU = 0, 1
SV_LOGITS, SV_PROBS = 0, 1
SV_Q2, SV_Q8 = 0, 1

EXPORTS = [
    "sv_api_version", "sv_status_str", "sv_q2_matrix_bytes", "sv_q2_tiled_bytes", "sv_q2_tile",
    "sv_q8_matrix_bytes",
    "sv_moe_workspace_bytes", "vq2_moe_gemm", "sv_lmhead_workspace_bytes", "vq8_lmhead_gemm",
    "sv_accept_workspace_bytes", "spec_accept", "spec_accept_noalloc", "vq2_dequant", "vq8_dequant",
    "sv_read_probe", "sv_accept_tsm_workspace_bytes", "spec_accept_target_sample", "sv_spec_account",
]


class SvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")


class MoeDesc(ctypes.Structure):
    _fields_ = [("ffn", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
                ("s_format", ctypes.c_int32)]


class SpecAccount(ctypes.Structure):
    """sv_spec_account_t: per-sequence step accounting of the yield-quench
    policy (zero-initialised before a request's first step)."""
    _fields_ = [("steps", ctypes.c_int64), ("tokens", ctypes.c_int64), ("regret", ctypes.c_double),
                ("quenched", ctypes.c_int32), ("quench_step", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None

_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_SIGS = {
    "sv_api_version": ([], ctypes.c_int),
    "sv_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "sv_q2_matrix_bytes": ([_i32, _i32], _sz),
    "sv_q2_tiled_bytes": ([_i32, _i32], _sz),
    "sv_q2_tile": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "sv_q8_matrix_bytes": ([_i32, _i32], _sz),
    "sv_moe_workspace_bytes": ([ctypes.POINTER(MoeDesc), _i32], _sz),
    "vq2_moe_gemm": ([ctypes.POINTER(MoeDesc), _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                     ctypes.c_int),
    "sv_lmhead_workspace_bytes": ([_i32, _i32], _sz),
    "vq8_lmhead_gemm": ([_vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "sv_accept_workspace_bytes": ([_i32, _i32, _i32], _sz),
    "spec_accept": ([_i32, _i32, _i32, _vp, _i32, _f32, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp,
                     _sz, _vp], ctypes.c_int),
    "spec_accept_noalloc": ([_i32, _i32, _i32, _vp, _i32, _f32, _vp, _i32, _f32, _vp, _vp, _vp, _vp,
                             _vp], ctypes.c_int),
    "vq2_dequant": ([_vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "vq8_dequant": ([_vp, _i32, _i32, _vp, _vp], ctypes.c_int),
    "sv_read_probe": ([_vp, _sz, _i32, _vp, _sz, _vp], ctypes.c_int),
    "sv_accept_tsm_workspace_bytes": ([_i32, _i32, _i32], _sz),
    "spec_accept_target_sample": ([_i32, _i32, _i32, _vp, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                                  ctypes.c_int),
    "sv_spec_account": ([_vp, _i32, _i32, ctypes.c_double, ctypes.c_double, ctypes.POINTER(SpecAccount)],
                        ctypes.c_int),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify.so (raises if it has not been built).

    torch is imported first: it carries its own HIP runtime under the same
    soname as the system one, and whichever is loaded first serves the whole
    process, so the library must bind to the runtime that owns torch's
    streams and allocations (loaded the other way round, every launch on a
    torch stream fails)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m bit_moe_tiny_amd.build` "
                          "(there is no fallback implementation)")
    import torch  # noqa: F401  (see above)
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().sv_status_str(int(status)).decode()


def api_version() -> int:
    return load().sv_api_version()


def _check(fn: str, st: int):
    if st != SV_OK:
        raise SvError(fn, st)


# ------------------------------------------------------------------ helpers
# Every tensor is checked against what the C ABI will read or write through
# its pointer (element type, shape, byte count) before the pointer is passed:
# a mismatch would otherwise be an out-of-bounds device access.
def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _act_dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise ValueError(f"activation rows must be float32 or bfloat16, not {t.dtype}")


def _want(t, name: str, dtype: str, shape=None, min_bytes: Optional[int] = None):
    """Checks tensor ``t`` (dtype one of 'f32', 'i32', 'u8', 'act' = f32 or
    bf16) against the shape / byte count the C call assumes."""
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    dts = {"f32": (torch.float32,), "i32": (torch.int32,), "u8": (torch.uint8, torch.int8),
           "act": (torch.float32, torch.bfloat16)}[dtype]
    if t.dtype not in dts:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dts)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, at least {min_bytes} needed")


def _dev_check(*ts):
    """Contiguous tensors on the current HIP device (checked after shapes)."""
    import torch
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if dev is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        if t.device != dev:
            raise ValueError(f"tensor on {t.device}, but the current device is {dev}")


def _workspace(nbytes: int, like):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=like.device)


# -------------------------------------------------------------------- sizes
def sv_q2_matrix_bytes(n_out: int, k_in: int) -> int:
    return load().sv_q2_matrix_bytes(n_out, k_in)


def sv_q8_matrix_bytes(n_out: int, k_in: int) -> int:
    return load().sv_q8_matrix_bytes(n_out, k_in)


def sv_q2_tiled_bytes(n_out: int, k_in: int) -> int:
    return load().sv_q2_tiled_bytes(n_out, k_in)


def sv_q2_tile(src, n_out: int, k_in: int, parts: int, count: int = 1, out=None, stream=None):
    """The `count` two-bit matrices [n_out x k_in] of the byte tensor ``src``
    (back to back) in the expert-tiled layout with `parts` K ranges (4 for
    gate and up, 1 for down); returns ``out`` (allocated when None)."""
    import torch
    a, b = sv_q2_matrix_bytes(n_out, k_in), sv_q2_tiled_bytes(n_out, k_in)
    if a == 0 or b == 0 or count < 1 or not 1 <= parts <= 64:
        raise ValueError(f"no tiled layout for {count} matrices [{n_out} x {k_in}], parts {parts}")
    _want(src, "src", "u8", min_bytes=count * a)
    if out is None:
        out = torch.empty(count * b, dtype=torch.uint8, device=src.device)
    _want(out, "out", "u8", min_bytes=count * b)
    _dev_check(src, out)
    _check("sv_q2_tile", load().sv_q2_tile(_ptr(src), _ptr(out), n_out, k_in, parts, count, _stream(stream)))
    return out


def _moe_weights(size, hidden, inter, n_experts, w_gate, w_up, w_down, s_gate, s_up, s_down, s_size=None):
    """The SwiGLU weight tensors hold the matrices the layer reads, `size`
    giving the bytes of one matrix in their layout (`s_size` that of the
    shared expert's, when its format differs)."""
    gu, dn = size(inter, hidden), size(hidden, inter)
    sgu, sdn = (gu, dn) if s_size is None else (s_size(inter, hidden), s_size(hidden, inter))
    if gu == 0 or dn == 0 or n_experts < 1:
        raise ValueError(f"no SwiGLU layer of hidden {hidden}, inter {inter}, {n_experts} experts")
    _want(w_gate, "w_gate", "u8", min_bytes=n_experts * gu)
    _want(w_up, "w_up", "u8", min_bytes=n_experts * gu)
    _want(w_down, "w_down", "u8", min_bytes=n_experts * dn)
    if s_gate is not None or s_up is not None or s_down is not None:
        if sgu == 0 or sdn == 0:
            raise ValueError(f"no shared expert of hidden {hidden}, inter {inter} in this format")
        _want(s_gate, "s_gate", "u8", min_bytes=sgu)
        _want(s_up, "s_up", "u8", min_bytes=sgu)
        _want(s_down, "s_down", "u8", min_bytes=sdn)
    _dev_check(w_gate, w_up, w_down, s_gate, s_up, s_down)


def moe_desc(ffn: int, hidden: int, inter: int, n_experts: int, top_k: int, w_gate, w_up=None,
             w_down=None, s_gate=None, s_up=None, s_down=None, tiled: bool = False,
             shared_format: int = SV_Q2) -> MoeDesc:
    """Layer description over device weight tensors (uint8 byte buffers), each
    checked to hold the matrices the layer reads: n_experts expert-major
    [inter x hidden] gate and up matrices and [hidden x inter] down matrices,
    one of each for the shared expert (PLAIN: w_gate alone, [inter x hidden]).
    SWIGLU weights are read in the expert-tiled layout: given in the plain
    layout (tiled=False) they are regrouped once here, on the device, by
    sv_q2_tile (gate and up with 4 parts, down with 1), and the description
    keeps the tiled copies alive.  shared_format SV_Q8: the shared expert's
    matrices are eight-bit (plain eight-bit layout, used as given)."""
    lib = load()
    gu = lib.sv_q2_matrix_bytes(inter, hidden)
    if ffn == SV_FFN_PLAIN:
        _want(w_gate, "w_gate", "u8", min_bytes=gu)
        if gu == 0:
            raise ValueError(f"no two-bit matrix of shape [{inter} x {hidden}]")
    else:
        if shared_format not in (SV_Q2, SV_Q8):
            raise ValueError(f"shared_format {shared_format}: expected SV_Q2 or SV_Q8")
        q8 = shared_format == SV_Q8
        s_size = lib.sv_q8_matrix_bytes if q8 else None
        if not tiled:
            _moe_weights(lib.sv_q2_matrix_bytes, hidden, inter, n_experts, w_gate, w_up, w_down, s_gate,
                         s_up, s_down, s_size)
            w_gate = sv_q2_tile(w_gate, inter, hidden, 4, n_experts)
            w_up = sv_q2_tile(w_up, inter, hidden, 4, n_experts)
            w_down = sv_q2_tile(w_down, hidden, inter, 1, n_experts)
            if not q8 and s_gate is not None and s_up is not None and s_down is not None:
                s_gate = sv_q2_tile(s_gate, inter, hidden, 4)
                s_up = sv_q2_tile(s_up, inter, hidden, 4)
                s_down = sv_q2_tile(s_down, hidden, inter, 1)
        _moe_weights(lib.sv_q2_tiled_bytes, hidden, inter, n_experts, w_gate, w_up, w_down, s_gate, s_up,
                     s_down, s_size)
    _dev_check(w_gate, w_up, w_down, s_gate, s_up, s_down)
    d = MoeDesc(ffn, hidden, inter, n_experts, top_k, _ptr(w_gate), _ptr(w_up), _ptr(w_down),
                _ptr(s_gate), _ptr(s_up), _ptr(s_down), shared_format if ffn != SV_FFN_PLAIN else SV_Q2)
    d._keep = (w_gate, w_up, w_down, s_gate, s_up, s_down)   # keep tensors alive
    return d


def sv_moe_workspace_bytes(desc: MoeDesc, R: int) -> int:
    return load().sv_moe_workspace_bytes(ctypes.byref(desc), R)


def sv_lmhead_workspace_bytes(hidden: int, R: int) -> int:
    return load().sv_lmhead_workspace_bytes(hidden, R)


def sv_accept_workspace_bytes(S: int, K: int, V: int) -> int:
    return load().sv_accept_workspace_bytes(S, K, V)


# ------------------------------------------------------------------- calls
def vq2_moe_gemm(desc: MoeDesc, x, router_logits, y, topk_idx=None, topk_w=None, ws=None,
                 stream=None):
    """y[R, hidden] (PLAIN: [R, inter]) from rows x[R, hidden] (fp32 or bf16)."""
    _want(x, "x", "act")
    if x.dim() != 2:
        raise ValueError(f"x: shape {tuple(x.shape)}, expected [R, {desc.hidden}]")
    R = x.shape[0]
    _want(x, "x", "act", (R, desc.hidden))
    plain = desc.ffn == SV_FFN_PLAIN
    _want(y, "y", "f32", (R, desc.inter if plain else desc.hidden))
    if router_logits is not None or (not plain and desc.n_experts > 1):
        _want(router_logits, "router_logits", "f32", (R, desc.n_experts))
    k = 1 if plain else desc.top_k
    if topk_idx is not None:
        _want(topk_idx, "topk_idx", "i32", (R, k))
    if topk_w is not None:
        _want(topk_w, "topk_w", "f32", (R, k))
    need = sv_moe_workspace_bytes(desc, R)
    if need == 0:
        raise ValueError(f"invalid layer description or row count R = {R}")
    if ws is not None:
        _want(ws, "ws", "u8", min_bytes=need)
    _dev_check(x, router_logits, y, topk_idx, topk_w, ws)
    if ws is None:
        ws = _workspace(need, x)
    st = load().vq2_moe_gemm(ctypes.byref(desc), _ptr(x), _act_dtype(x), R, _ptr(router_logits),
                             _ptr(y), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check("vq2_moe_gemm", st)
    return y


def vq8_lmhead_gemm(w, vocab: int, hidden: int, h, logits, ws=None, stream=None):
    """logits[R, vocab] from hidden rows h[R, hidden] (fp32 or bf16)."""
    _want(w, "w", "u8", min_bytes=max(sv_q8_matrix_bytes(vocab, hidden), 1))
    _want(h, "h", "act")
    if h.dim() != 2:
        raise ValueError(f"h: shape {tuple(h.shape)}, expected [R, {hidden}]")
    R = h.shape[0]
    _want(h, "h", "act", (R, hidden))
    _want(logits, "logits", "f32", (R, vocab))
    need = sv_lmhead_workspace_bytes(hidden, R)
    if need == 0 or sv_q8_matrix_bytes(vocab, hidden) == 0:
        raise ValueError(f"invalid head shape vocab {vocab} x hidden {hidden} or row count R = {R}")
    if ws is not None:
        _want(ws, "ws", "u8", min_bytes=need)
    _dev_check(w, h, logits, ws)
    if ws is None:
        ws = _workspace(need, h)
    st = load().vq8_lmhead_gemm(_ptr(w), vocab, hidden, _ptr(h), _act_dtype(h), R, _ptr(logits),
                                _ptr(ws), ws.numel(), _stream(stream))
    _check("vq8_lmhead_gemm", st)
    return logits


def spec_accept(S: int, K: int, V: int, target, target_kind: int, t_p: float, draft,
                draft_kind: int, t_q: float, draft_tokens, uniforms, out_tokens, out_n_accepted,
                ws=None, stream=None):
    """Accept/reject for S sequences of K drafts; fills out_tokens [S, K+1] and
    out_n_accepted [S] (int32).  A logits row at temperature 0 is greedy: the
    one-hot distribution at its first largest value."""
    need = sv_accept_workspace_bytes(S, K, V)
    if need == 0:
        raise ValueError(f"invalid accept shape S = {S}, K = {K}, V = {V}")
    _want(target, "target", "f32", (S * (K + 1), V))
    if K > 0:
        _want(draft, "draft", "f32", (S * K, V))
        _want(draft_tokens, "draft_tokens", "i32", (S, K))
    _want(uniforms, "uniforms", "f32", (S, K + 1))
    _want(out_tokens, "out_tokens", "i32", (S, K + 1))
    _want(out_n_accepted, "out_n_accepted", "i32", (S,))
    if ws is not None:
        _want(ws, "ws", "u8", min_bytes=need)
    _dev_check(target, draft, draft_tokens, uniforms, out_tokens, out_n_accepted, ws)
    if ws is None:
        ws = _workspace(need, target)
    st = load().spec_accept(S, K, V, _ptr(target), target_kind, t_p, _ptr(draft), draft_kind, t_q,
                            _ptr(draft_tokens), _ptr(uniforms), _ptr(out_tokens),
                            _ptr(out_n_accepted), _ptr(ws), ws.numel(), _stream(stream))
    _check("spec_accept", st)
    return out_tokens, out_n_accepted


def spec_accept_noalloc(S: int, K: int, V: int, target, target_kind: int, t_p: float, draft,
                        draft_kind: int, t_q: float, draft_tokens, uniforms, out_tokens,
                        out_n_accepted, stream=None):
    """spec_accept on the library's static scratch array: no workspace, no
    allocation (for callers that cannot allocate, e.g. under graph capture).
    Calls that overlap on one GPU race; raises SvError(SV_ESCRATCH) when the
    shape needs more than the array holds."""
    if sv_accept_workspace_bytes(S, K, V) == 0:
        raise ValueError(f"invalid accept shape S = {S}, K = {K}, V = {V}")
    _want(target, "target", "f32", (S * (K + 1), V))
    if K > 0:
        _want(draft, "draft", "f32", (S * K, V))
        _want(draft_tokens, "draft_tokens", "i32", (S, K))
    _want(uniforms, "uniforms", "f32", (S, K + 1))
    _want(out_tokens, "out_tokens", "i32", (S, K + 1))
    _want(out_n_accepted, "out_n_accepted", "i32", (S,))
    _dev_check(target, draft, draft_tokens, uniforms, out_tokens, out_n_accepted)
    st = load().spec_accept_noalloc(S, K, V, _ptr(target), target_kind, t_p, _ptr(draft), draft_kind,
                                    t_q, _ptr(draft_tokens), _ptr(uniforms), _ptr(out_tokens),
                                    _ptr(out_n_accepted), _stream(stream))
    _check("spec_accept_noalloc", st)
    return out_tokens, out_n_accepted


def sv_accept_tsm_workspace_bytes(S: int, K: int, V: int) -> int:
    return load().sv_accept_tsm_workspace_bytes(S, K, V)


def spec_accept_target_sample(S: int, K: int, V: int, target, target_kind: int, t_p: float,
                              draft_tokens, uniforms, out_tokens, out_n_accepted, ws=None, stream=None):
    """Target-sample matching for S sequences of K drafts: every verify row's
    own sample at its uniform, drafts kept while they match; fills out_tokens
    [S, K+1] and out_n_accepted [S] (int32).  No draft distribution."""
    need = sv_accept_tsm_workspace_bytes(S, K, V)
    if need == 0:
        raise ValueError(f"invalid accept shape S = {S}, K = {K}, V = {V}")
    _want(target, "target", "f32", (S * (K + 1), V))
    if K > 0:
        _want(draft_tokens, "draft_tokens", "i32", (S, K))
    _want(uniforms, "uniforms", "f32", (S, K + 1))
    _want(out_tokens, "out_tokens", "i32", (S, K + 1))
    _want(out_n_accepted, "out_n_accepted", "i32", (S,))
    if ws is not None:
        _want(ws, "ws", "u8", min_bytes=need)
    _dev_check(target, draft_tokens if K > 0 else None, uniforms, out_tokens, out_n_accepted, ws)
    if ws is None:
        ws = _workspace(need, target)
    st = load().spec_accept_target_sample(S, K, V, _ptr(target), target_kind, t_p,
                                          _ptr(draft_tokens) if K > 0 else None, _ptr(uniforms),
                                          _ptr(out_tokens), _ptr(out_n_accepted), _ptr(ws), ws.numel(),
                                          _stream(stream))
    _check("spec_accept_target_sample", st)
    return out_tokens, out_n_accepted


def sv_spec_account(n_accepted, K: int, guard: float, threshold: float, state=None):
    """One verify step of the yield-quench accounting (host): n_accepted is a
    host sequence of S int32 values as an accept call wrote them; ``state`` a
    ctypes array of S SpecAccount (created zeroed when None).  Returns
    ``state``."""
    import numpy as np
    n = np.ascontiguousarray(np.asarray(n_accepted, dtype=np.int32).reshape(-1))
    S = int(n.shape[0])
    if state is None:
        state = (SpecAccount * S)()
    if len(state) != S:
        raise ValueError(f"state holds {len(state)} sequences, n_accepted {S}")
    _check("sv_spec_account", load().sv_spec_account(n.ctypes.data, S, K, float(guard), float(threshold),
                                                     ctypes.cast(state, ctypes.POINTER(SpecAccount))))
    return state


def vq2_dequant(w, n_out: int, k_in: int, out, stream=None):
    nb = sv_q2_matrix_bytes(n_out, k_in)
    if nb == 0:
        raise ValueError(f"no two-bit matrix of shape [{n_out} x {k_in}]")
    _want(w, "w", "u8", min_bytes=nb)
    _want(out, "out", "f32", (n_out, k_in))
    _dev_check(w, out)
    _check("vq2_dequant", load().vq2_dequant(_ptr(w), n_out, k_in, _ptr(out), _stream(stream)))
    return out


def vq8_dequant(w, n_out: int, k_in: int, out, stream=None):
    nb = sv_q8_matrix_bytes(n_out, k_in)
    if nb == 0:
        raise ValueError(f"no eight-bit matrix of shape [{n_out} x {k_in}]")
    _want(w, "w", "u8", min_bytes=nb)
    _want(out, "out", "f32", (n_out, k_in))
    _dev_check(w, out)
    _check("vq8_dequant", load().vq8_dequant(_ptr(w), n_out, k_in, _ptr(out), _stream(stream)))
    return out


PROBE_GROUP_BYTES = 16 * 1792   # SV_PROBE_GROUP_BYTES of the header


def sv_read_probe(src, mode: int, sink, stream=None):
    """Reads the byte buffer ``src`` once in access pattern ``mode`` (0..3; see
    the header); ``sink`` is an int32 device tensor of at least 8 words per
    compute unit.  Returns the number of bytes read."""
    _want(src, "src", "u8", min_bytes=PROBE_GROUP_BYTES)
    _want(sink, "sink", "i32")
    _dev_check(src, sink)
    _check("sv_read_probe", load().sv_read_probe(_ptr(src), src.numel(), mode, _ptr(sink), sink.numel(),
                                                 _stream(stream)))
    return src.numel() // PROBE_GROUP_BYTES * PROBE_GROUP_BYTES
