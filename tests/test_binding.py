"""The Python binding checks every tensor against what the C call will read or
write through its pointer (element type, shape, byte count) and raises
ValueError before any pointer is passed.  CPU tensors stand in for device
tensors: the shape checks come before the device check, so every case here
raises before anything reaches the library's compute entry points."""
import pytest
import torch

import bit_moe_tiny_amd as sv

H, I, E, K = 512, 256, 8, 2


def _f32(*s):
    return torch.zeros(s, dtype=torch.float32)


def _i32(*s):
    return torch.zeros(s, dtype=torch.int32)


def _bf16(*s):
    return torch.zeros(s, dtype=torch.bfloat16)


def _desc(ffn=sv.SV_FFN_SWIGLU, n_experts=E, top_k=K):
    # pointers are never dereferenced: every call below fails validation first
    return sv.MoeDesc(ffn, H, I, n_experts, top_k, 16, 16, 16, 0, 0, 0)


def _raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_moe_desc_checks_weight_sizes():
    gu = sv.sv_q2_matrix_bytes(I, H)
    dn = sv.sv_q2_matrix_bytes(H, I)
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    _raises("w_gate", sv.moe_desc, sv.SV_FFN_SWIGLU, H, I, E, K, u8(E * gu - 1), u8(E * gu), u8(E * dn))
    _raises("w_down", sv.moe_desc, sv.SV_FFN_SWIGLU, H, I, E, K, u8(E * gu), u8(E * gu), u8(E * dn - 1))
    _raises("s_up", sv.moe_desc, sv.SV_FFN_SWIGLU, H, I, E, K, u8(E * gu), u8(E * gu), u8(E * dn),
            u8(gu), u8(gu - 1), u8(dn))
    _raises("w_up", sv.moe_desc, sv.SV_FFN_SWIGLU, H, I, E, K, u8(E * gu), _f32(E * gu), u8(E * dn))
    _raises("no SwiGLU layer", sv.moe_desc, sv.SV_FFN_SWIGLU, 500, I, E, K, u8(1), u8(1), u8(1))
    # right sizes, but host memory: the device check refuses them
    _raises("device", sv.moe_desc, sv.SV_FFN_SWIGLU, H, I, E, K, u8(E * gu), u8(E * gu), u8(E * dn))


@pytest.mark.parametrize("case", ["x_dtype", "x_shape", "y_shape", "y_dtype", "logits_dtype",
                                  "logits_shape", "logits_missing", "idx_dtype", "w_shape",
                                  "ws_small", "rows"])
def test_vq2_moe_gemm_checks(case):
    R = 5
    a = dict(x=_bf16(R, H), router_logits=_f32(R, E), y=_f32(R, H), topk_idx=_i32(R, K),
             topk_w=_f32(R, K))
    want = {"x_dtype": "x", "x_shape": "x", "y_shape": "y", "y_dtype": "y",
            "logits_dtype": "router_logits", "logits_shape": "router_logits",
            "logits_missing": "router_logits", "idx_dtype": "topk_idx", "w_shape": "topk_w",
            "ws_small": "ws", "rows": "row count"}[case]
    if case == "x_dtype":
        a["x"] = torch.zeros((R, H), dtype=torch.float16)
    elif case == "x_shape":
        a["x"] = _bf16(R, H + 256)
    elif case == "y_shape":
        a["y"] = _f32(R, I)
    elif case == "y_dtype":
        a["y"] = _bf16(R, H)
    elif case == "logits_dtype":
        a["router_logits"] = _bf16(R, E)
    elif case == "logits_shape":
        a["router_logits"] = _f32(R, E + 1)
    elif case == "logits_missing":
        a["router_logits"] = None
    elif case == "idx_dtype":
        a["topk_idx"] = torch.zeros((R, K), dtype=torch.int64)
    elif case == "w_shape":
        a["topk_w"] = _f32(R, K + 1)
    elif case == "ws_small":
        a["ws"] = torch.zeros(16, dtype=torch.uint8)
    elif case == "rows":
        R = 65
        a.update(x=_bf16(R, H), router_logits=_f32(R, E), y=_f32(R, H), topk_idx=None, topk_w=None)
    _raises(want, sv.vq2_moe_gemm, _desc(), **a)


def test_vq2_moe_gemm_plain_output_shape():
    d = sv.MoeDesc(sv.SV_FFN_PLAIN, H, I, 1, 1, 16, 0, 0, 0, 0, 0)
    _raises("y", sv.vq2_moe_gemm, d, _f32(3, H), None, _f32(3, H))   # PLAIN writes [R, inter]
    _raises("device", sv.vq2_moe_gemm, d, _f32(3, H), None, _f32(3, I))


def test_vq8_lmhead_gemm_checks():
    V, Hd, R = 1000, 1024, 4
    w = torch.zeros(sv.sv_q8_matrix_bytes(V, Hd), dtype=torch.uint8)
    _raises("w", sv.vq8_lmhead_gemm, w[:-1], V, Hd, _bf16(R, Hd), _f32(R, V))
    _raises("h", sv.vq8_lmhead_gemm, w, V, Hd, _bf16(R, Hd - 32), _f32(R, V))
    _raises("h", sv.vq8_lmhead_gemm, w, V, Hd, torch.zeros((R, Hd), dtype=torch.float64), _f32(R, V))
    _raises("logits", sv.vq8_lmhead_gemm, w, V, Hd, _bf16(R, Hd), _f32(R, V - 1))
    _raises("logits", sv.vq8_lmhead_gemm, w, V, Hd, _bf16(R, Hd), _bf16(R, V))
    _raises("ws", sv.vq8_lmhead_gemm, w, V, Hd, _bf16(R, Hd), _f32(R, V), ws=torch.zeros(8, dtype=torch.uint8))
    _raises("row count", sv.vq8_lmhead_gemm, w, V, Hd, _bf16(65, Hd), _f32(65, V))
    _raises("device", sv.vq8_lmhead_gemm, w, V, Hd, _bf16(R, Hd), _f32(R, V))


@pytest.mark.parametrize("case", ["target", "draft", "tokens_dtype", "tokens_shape", "uniforms",
                                  "uniforms_dtype", "out_tokens", "out_n", "ws", "shape"])
def test_spec_accept_checks(case):
    S, K, V = 2, 3, 100
    a = dict(target=_f32(S * (K + 1), V), draft=_f32(S * K, V), draft_tokens=_i32(S, K),
             uniforms=_f32(S, K + 1), out_tokens=_i32(S, K + 1), out_n_accepted=_i32(S))
    want = case
    if case == "target":
        a["target"] = _f32(S * K, V)
    elif case == "draft":
        a["draft"] = _f32(S * K, V + 1)
    elif case == "tokens_dtype":
        a["draft_tokens"] = torch.zeros((S, K), dtype=torch.int64)
        want = "draft_tokens"
    elif case == "tokens_shape":
        a["draft_tokens"] = _i32(S, K + 1)
        want = "draft_tokens"
    elif case == "uniforms":
        a["uniforms"] = _f32(S, K)
    elif case == "uniforms_dtype":
        a["uniforms"] = torch.zeros((S, K + 1), dtype=torch.float64)
        want = "uniforms"
    elif case == "out_tokens":
        a["out_tokens"] = _i32(S, K)
    elif case == "out_n":
        a["out_n_accepted"] = _i32(S + 1)
        want = "out_n_accepted"
    elif case == "ws":
        a["ws"] = torch.zeros(8, dtype=torch.uint8)
    elif case == "shape":
        K = 40   # beyond the draft limit
        want = "invalid accept shape"
    _raises(want, sv.spec_accept, S, K, V, a["target"], sv.SV_LOGITS, 1.0, a["draft"], sv.SV_LOGITS, 1.0,
            a["draft_tokens"], a["uniforms"], a["out_tokens"], a["out_n_accepted"], ws=a.get("ws"))


def test_spec_accept_without_drafts_needs_no_draft_tensors():
    S, V = 2, 100
    _raises("device", sv.spec_accept, S, 0, V, _f32(S, V), sv.SV_LOGITS, 1.0, None, sv.SV_LOGITS, 1.0,
            None, _f32(S, 1), _i32(S, 1), _i32(S))


def test_dequant_checks():
    n, k = 64, 512
    w2 = torch.zeros(sv.sv_q2_matrix_bytes(n, k), dtype=torch.uint8)
    _raises("w", sv.vq2_dequant, w2[:-1], n, k, _f32(n, k))
    _raises("out", sv.vq2_dequant, w2, n, k, _f32(n, k - 1))
    _raises("no two-bit", sv.vq2_dequant, w2, n, 100, _f32(n, 100))
    w8 = torch.zeros(sv.sv_q8_matrix_bytes(n, k), dtype=torch.uint8)
    _raises("w", sv.vq8_dequant, w8[:-1], n, k, _f32(n, k))
    _raises("out", sv.vq8_dequant, w8, n, k, _bf16(n, k))
    _raises("device", sv.vq8_dequant, w8, n, k, _f32(n, k))
