"""The C-ABI library loads, exports every declared symbol, and validates
arguments on the host (CPU only: every call here returns before any launch)."""
import ctypes
import os
import re

import pytest

import bit_moe_tiny_amd as sv
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared():
    txt = open(HEADER).read()
    return re.findall(r"SV_API\s+[\w\s\*]+?\b(\w+)\s*\(", txt)


def test_library_exports_every_declared_symbol():
    lib = sv.load()
    names = _declared()
    assert len(names) == 19
    assert set(names) == set(sv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    # nothing beyond the C ABI is exported
    out = os.popen(f"nm -D --defined-only {sv.LIB_PATH}").read()
    text_syms = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert text_syms == set(names)


def test_version_and_status_strings():
    assert sv.api_version() == 3
    assert sv.status_str(sv.SV_OK) == "ok"
    assert "workspace" in sv.status_str(sv.SV_EWORKSPACE)
    assert sv.status_str(99) == "unknown status"


@pytest.mark.parametrize("n,k", [(2048, 7168), (7168, 2048), (512, 256), (1, 256), (13, 768)])
def test_q2_matrix_bytes_agree_with_oracle(n, k):
    assert sv.sv_q2_matrix_bytes(n, k) == oracle.q2_matrix_bytes(n, k)


@pytest.mark.parametrize("n,k", [(129280, 7168), (1, 32), (7, 64)])
def test_q8_matrix_bytes_agree_with_oracle(n, k):
    assert sv.sv_q8_matrix_bytes(n, k) == oracle.q8_matrix_bytes(n, k)


@pytest.mark.parametrize("n,k", [(2048, 7168), (7168, 2048), (16, 256), (48, 768)])
def test_q2_tiled_bytes_are_84_per_256_weights(n, k):
    assert sv.sv_q2_tiled_bytes(n, k) == 84 * n * k // 256


def test_q2_tiled_bytes_reject_invalid_shapes():
    for n, k in ((8, 256), (24, 256), (0, 256), (16, 100), (16, 0)):
        assert sv.sv_q2_tiled_bytes(n, k) == 0, (n, k)


def test_q2_tile_validates_on_the_host():
    lib = sv.load()
    a, b = 0x10000000, 0x20000000
    assert lib.sv_q2_tile(None, b, 32, 512, 4, 1, None) == sv.SV_EINVAL
    assert lib.sv_q2_tile(a, None, 32, 512, 4, 1, None) == sv.SV_EINVAL
    assert lib.sv_q2_tile(a, b, 24, 512, 4, 1, None) == sv.SV_EINVAL      # rows not a multiple of 16
    assert lib.sv_q2_tile(a, b, 32, 500, 4, 1, None) == sv.SV_EINVAL
    assert lib.sv_q2_tile(a, b, 32, 512, 0, 1, None) == sv.SV_EINVAL
    assert lib.sv_q2_tile(a, b, 32, 512, 65, 1, None) == sv.SV_EINVAL
    assert lib.sv_q2_tile(a, b, 32, 512, 4, 0, None) == sv.SV_EINVAL
    assert lib.sv_q2_tile(a, a + 64, 32, 512, 4, 1, None) == sv.SV_EINVAL  # overlapping buffers


def test_invalid_shapes_give_zero_sizes():
    assert sv.sv_q2_matrix_bytes(10, 100) == 0 and sv.sv_q2_matrix_bytes(0, 256) == 0
    assert sv.sv_q8_matrix_bytes(10, 33) == 0
    assert sv.sv_lmhead_workspace_bytes(7168, 0) == 0 and sv.sv_lmhead_workspace_bytes(7168, 65) == 0
    assert sv.sv_lmhead_workspace_bytes(100, 4) == 0
    assert sv.sv_accept_workspace_bytes(1, 32, 100) == 0 and sv.sv_accept_workspace_bytes(0, 4, 100) == 0
    assert sv.sv_accept_workspace_bytes(1, 4, 600000) == 0
    assert sv.sv_accept_workspace_bytes(3, 4, 129280) > 0


def _desc(**kw):
    base = dict(ffn=sv.SV_FFN_SWIGLU, hidden=7168, inter=2048, n_experts=256, top_k=8)
    base.update(kw)
    d = sv.MoeDesc(base["ffn"], base["hidden"], base["inter"], base["n_experts"], base["top_k"],
                   base.get("w_gate", 0x1000), base.get("w_up", 0x1000), base.get("w_down", 0x1000),
                   base.get("s_gate"), base.get("s_up"), base.get("s_down"), base.get("s_format", 0))
    return d


def test_moe_workspace_sizes():
    assert sv.sv_moe_workspace_bytes(_desc(), 5) > 0
    assert sv.sv_moe_workspace_bytes(_desc(s_gate=1, s_up=1, s_down=1), 16) > sv.sv_moe_workspace_bytes(_desc(), 16)
    assert sv.sv_moe_workspace_bytes(_desc(), 0) == 0
    assert sv.sv_moe_workspace_bytes(_desc(), 65) == 0
    assert sv.sv_moe_workspace_bytes(_desc(hidden=7000), 5) == 0
    assert sv.sv_moe_workspace_bytes(_desc(top_k=17), 5) == 0
    assert sv.sv_moe_workspace_bytes(_desc(top_k=9, n_experts=8), 5) == 0
    assert sv.sv_moe_workspace_bytes(_desc(s_gate=1), 5) == 0          # shared expert all-or-none
    assert sv.sv_moe_workspace_bytes(_desc(ffn=sv.SV_FFN_PLAIN, inter=512, hidden=256, n_experts=1,
                                           top_k=1, w_up=None, w_down=None), 4) > 0
    assert sv.sv_moe_workspace_bytes(_desc(ffn=7), 4) == 0
    # the shared expert's format: SV_Q2 or SV_Q8 (eight-bit needs its staging and output space)
    assert sv.sv_moe_workspace_bytes(_desc(s_gate=1, s_up=1, s_down=1, s_format=2), 5) == 0
    q2s = sv.sv_moe_workspace_bytes(_desc(s_gate=1, s_up=1, s_down=1, s_format=sv.SV_Q2), 5)
    q8s = sv.sv_moe_workspace_bytes(_desc(s_gate=1, s_up=1, s_down=1, s_format=sv.SV_Q8), 5)
    assert q8s > q2s > 0
    assert sv.sv_moe_workspace_bytes(_desc(s_format=5), 5) > 0      # ignored without a shared expert


def test_calls_reject_bad_arguments_before_launch():
    lib = sv.load()
    d = _desc()
    fake = ctypes.c_void_p(0x1000)
    # R out of range, missing router, null output, bad dtype: all EINVAL, no launch
    assert lib.vq2_moe_gemm(ctypes.byref(d), fake, 1, 0, fake, fake, None, None, fake, 1 << 30, None) == sv.SV_EINVAL
    assert lib.vq2_moe_gemm(ctypes.byref(d), fake, 1, 5, None, fake, None, None, fake, 1 << 30, None) == sv.SV_EINVAL
    assert lib.vq2_moe_gemm(ctypes.byref(d), fake, 1, 5, fake, None, None, None, fake, 1 << 30, None) == sv.SV_EINVAL
    assert lib.vq2_moe_gemm(ctypes.byref(d), fake, 7, 5, fake, fake, None, None, fake, 1 << 30, None) == sv.SV_EINVAL
    # undersized workspace
    assert lib.vq2_moe_gemm(ctypes.byref(d), fake, 1, 5, fake, fake, None, None, fake, 16, None) == sv.SV_EWORKSPACE
    assert lib.vq8_lmhead_gemm(fake, 129280, 7168, fake, 1, 5, fake, fake, 16, None) == sv.SV_EWORKSPACE
    assert lib.vq8_lmhead_gemm(fake, 0, 7168, fake, 1, 5, fake, fake, 1 << 30, None) == sv.SV_EINVAL
    assert lib.vq8_lmhead_gemm(fake, 100, 7168, fake, 1, 65, fake, fake, 1 << 30, None) == sv.SV_EINVAL
    # accept: bad temperature, bad kind, missing drafts, undersized workspace
    args = lambda **k: [k.get("S", 1), k.get("K", 4), k.get("V", 32), fake, k.get("tk", 0),
                        k.get("tp", 1.0), k.get("draft", fake), k.get("dk", 0), k.get("tq", 1.0),
                        k.get("tok", fake), fake, fake, fake, fake, k.get("wsb", 1 << 20), None]
    assert lib.spec_accept(*args(tp=-0.5)) == sv.SV_EINVAL
    assert lib.spec_accept(*args(tq=float("nan"))) == sv.SV_EINVAL
    assert lib.spec_accept(*args(tk=3)) == sv.SV_EINVAL
    assert lib.spec_accept(*args(draft=None)) == sv.SV_EINVAL
    assert lib.spec_accept(*args(tok=None)) == sv.SV_EINVAL
    assert lib.spec_accept(*args(K=32)) == sv.SV_EINVAL
    assert lib.spec_accept(*args(wsb=8)) == sv.SV_EWORKSPACE
    # the allocation-free variant: the same argument checks, and shapes whose
    # scratch need exceeds the static array are refused before any HIP call
    nargs = lambda **k: args(**k)[:13] + [None]
    assert lib.spec_accept_noalloc(*nargs(tp=-0.5)) == sv.SV_EINVAL
    assert lib.spec_accept_noalloc(*nargs(draft=None)) == sv.SV_EINVAL
    assert lib.spec_accept_noalloc(*nargs(K=32)) == sv.SV_EINVAL
    assert sv.sv_accept_workspace_bytes(40, 4, 129280) > sv.ACCEPT_SCRATCH_BYTES
    assert sv.sv_accept_workspace_bytes(31, 4, 129280) <= sv.ACCEPT_SCRATCH_BYTES
    assert lib.spec_accept_noalloc(*nargs(S=40, V=129280)) == sv.SV_ESCRATCH
    assert "scratch" in sv.status_str(sv.SV_ESCRATCH)
    assert lib.sv_read_probe(fake, 1 << 20, 6, fake, 1 << 16, None) == sv.SV_EINVAL
    assert lib.sv_read_probe(fake, 100, 0, fake, 1 << 16, None) == sv.SV_EINVAL
    assert lib.vq2_dequant(fake, 10, 100, fake, None) == sv.SV_EINVAL
    assert lib.vq8_dequant(fake, 10, 33, fake, None) == sv.SV_EINVAL
    # target-sample matching: the same shape, kind, temperature and workspace checks
    targs = lambda **k: [k.get("S", 1), k.get("K", 4), k.get("V", 32), k.get("target", fake),
                         k.get("tk", 0), k.get("tp", 1.0), k.get("tok", fake), fake, fake, fake,
                         k.get("ws", fake), k.get("wsb", 1 << 20), None]
    assert lib.spec_accept_target_sample(*targs(tp=-1.0)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(tp=float("inf"))) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(tk=2)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(tok=None)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(target=None)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(ws=None)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(K=32)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(V=0)) == sv.SV_EINVAL
    assert lib.spec_accept_target_sample(*targs(wsb=8)) == sv.SV_EWORKSPACE
    assert sv.sv_accept_tsm_workspace_bytes(1, 0, 1) > 0
    assert sv.sv_accept_tsm_workspace_bytes(0, 4, 32) == 0
    assert sv.sv_accept_tsm_workspace_bytes(1, 4, 256 * 2048 + 1) == 0


def test_spec_account_matches_the_oracle():
    """The host accounting against oracle.yield_quench, step by step, on
    random runs of accepted-draft counts (with invalid -1 steps); fp64 on
    both sides in the same order, so the regrets agree exactly."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(17)
    S, K, steps = 64, 4, 40
    guard, th = 2.16, 4.0
    p_acc = rng.uniform(0.2, 0.95, size=S)
    runs = np.where(rng.random((steps, S)) < 0.05, -1,
                    np.minimum(rng.geometric(1 - p_acc[None, :], size=(steps, S)) - 1, K)).astype(np.int32)
    state = None
    for k in range(steps):
        state = sv.sv_spec_account(runs[k], K, guard, th, state)
    quenched = 0
    for s in range(S):
        st, tok, reg, q = oracle.yield_quench(runs[:, s].tolist(), guard, th)
        a = state[s]
        assert (a.steps, a.tokens, a.regret) == (st, tok, reg), s
        assert a.quenched == (q is not None) and a.quench_step == (q or 0), s
        quenched += a.quenched
    assert 0 < quenched < S


def test_spec_account_rejects_bad_arguments():
    import numpy as np
    lib = sv.load()
    st = (sv.SpecAccount * 2)()
    st[0].regret = 1.5
    n = np.array([1, 5], np.int32)
    ptr = ctypes.cast(st, ctypes.POINTER(sv.SpecAccount))
    assert lib.sv_spec_account(n.ctypes.data, 2, 4, 2.16, 4.0, ptr) == sv.SV_EINVAL   # 5 > K
    assert st[0].regret == 1.5 and st[0].steps == 0                                     # nothing changed
    n[1] = -2
    assert lib.sv_spec_account(n.ctypes.data, 2, 4, 2.16, 4.0, ptr) == sv.SV_EINVAL
    n[1] = -1
    assert lib.sv_spec_account(n.ctypes.data, 2, 4, float("nan"), 4.0, ptr) == sv.SV_EINVAL
    assert lib.sv_spec_account(n.ctypes.data, 2, 4, 2.16, float("inf"), ptr) == sv.SV_EINVAL
    assert lib.sv_spec_account(n.ctypes.data, 0, 4, 2.16, 4.0, ptr) == sv.SV_EINVAL
    assert lib.sv_spec_account(n.ctypes.data, 2, 32, 2.16, 4.0, ptr) == sv.SV_EINVAL
    assert lib.sv_spec_account(None, 2, 4, 2.16, 4.0, ptr) == sv.SV_EINVAL
    assert lib.sv_spec_account(n.ctypes.data, 2, 4, 2.16, 4.0, None) == sv.SV_EINVAL
    assert lib.sv_spec_account(n.ctypes.data, 2, 4, 2.16, 4.0, ptr) == sv.SV_OK
    assert (st[0].steps, st[0].tokens, st[1].steps) == (1, 2, 0)
    assert st[0].regret == 1.5 + (2.16 - 2)


def test_binding_has_no_fallback(tmp_path):
    from bit_moe_tiny_amd import _lib
    saved = _lib._lib
    _lib._lib = None
    try:
        with pytest.raises(ImportError):
            _lib.load(str(tmp_path / "missing.so"))
    finally:
        _lib._lib = saved
