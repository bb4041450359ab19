"""libspecverify for MI355X: the verifier step of lossless speculative decoding
over a two-bit MoE, as hand-written HIP kernels behind a C ABI.

The Python names mirror the C ABI (``include/specverify.h``); they only
marshal arguments.  Build the library with ``python -m bit_moe_tiny_amd.build``.
"""
from ._lib import (ACCEPT_SCRATCH_BYTES, EXPORTS, LIB_PATH, MoeDesc, SV_BF16, SV_EHIP, SV_EINVAL,
                   SV_ESCRATCH, SV_EUNSUPPORTED, SV_EWORKSPACE, SV_F32, SV_FFN_PLAIN,
                   SV_FFN_SWIGLU, SV_LOGITS, SV_OK, SV_PROBS, SvError, api_version, load, moe_desc,
                   spec_accept, spec_accept_noalloc, sv_read_probe, PROBE_GROUP_BYTES,
                   SpecAccount, spec_accept_target_sample, sv_accept_tsm_workspace_bytes,
                   sv_spec_account, SV_Q2, SV_Q8,
                   status_str, sv_accept_workspace_bytes, sv_lmhead_workspace_bytes,
                   sv_moe_workspace_bytes, sv_q2_matrix_bytes, sv_q2_tile, sv_q2_tiled_bytes,
                   sv_q8_matrix_bytes, vq2_dequant,
                   vq2_moe_gemm, vq8_dequant, vq8_lmhead_gemm)

__all__ = [
    "EXPORTS", "LIB_PATH", "MoeDesc", "SvError", "load", "api_version", "status_str", "moe_desc",
    "sv_q2_matrix_bytes", "sv_q2_tiled_bytes", "sv_q2_tile", "sv_q8_matrix_bytes", "sv_moe_workspace_bytes",
    "sv_lmhead_workspace_bytes", "sv_accept_workspace_bytes", "vq2_moe_gemm",
    "vq8_lmhead_gemm", "spec_accept", "spec_accept_noalloc", "vq2_dequant", "vq8_dequant",
    "sv_read_probe", "PROBE_GROUP_BYTES",
    "SpecAccount", "spec_accept_target_sample", "sv_accept_tsm_workspace_bytes", "sv_spec_account",
    "SV_Q2", "SV_Q8",
    "ACCEPT_SCRATCH_BYTES", "SV_OK", "SV_EINVAL", "SV_EUNSUPPORTED", "SV_EWORKSPACE", "SV_EHIP",
    "SV_ESCRATCH", "SV_F32", "SV_BF16",
    "SV_FFN_PLAIN", "SV_FFN_SWIGLU", "SV_LOGITS", "SV_PROBS",
]
