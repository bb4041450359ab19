"""The verifier step captured as a HIP graph (torch.cuda.CUDAGraph over the
C-ABI calls, which only launch kernels): every replay gives bit-identical
outputs to the eager run of the same inputs, also when the program's own
eager work on other inputs -- which overwrites every output and workspace
the graph uses -- runs between the replays, with synchronisations between.

The step: two stacked MoE layers at the full expert shape (7168 <-> 2048,
16 routed experts + the shared one, top-8), each preceded by its eight-bit
router GEMV, then an eight-bit head (2048 x 7168) and spec_accept (S = 1,
K = R - 1)."""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

H, I, E, TOPK, V, L = synth.HIDDEN, synth.INTER, 16, synth.TOP_K, 2048, 2


@pytest.fixture(scope="module")
def sv():
    import bit_moe_tiny_amd as m
    m.load()
    return m


@pytest.fixture(scope="module")
def model(sv):
    say("generating 17 experts, a router and a head")
    mats = [synth.expert_matrices(synth.CFG_MOE, e) for e in range(E + 1)]
    cat = lambda m: np.concatenate([mats[e][m].packed() for e in range(E)])
    t = [dev(cat(m)) for m in (synth.M_GATE, synth.M_UP, synth.M_DOWN)]
    t += [dev(mats[E][m].packed()) for m in (synth.M_GATE, synth.M_UP, synth.M_DOWN)]
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, H, I, E, TOPK, *t)
    wr = dev(synth.q8_random(synth.generator(synth.CFG_MOE, 77), E, H, 0.01).packed())
    wh = dev(synth.q8_random(synth.generator(synth.CFG_LMHEAD, 77), V, H, 0.01).packed())
    return desc, wr, wh


class Stack:
    def __init__(self, sv, model, R):
        import torch
        self.sv, (self.desc, self.wr, self.wh) = sv, model
        self.R, self.K = R, R - 1
        f = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
        self.x = dev(synth.moe_rows(R, synth.CFG_MOE, sub=700 + R).x_bf16)
        self.ys, self.lg = [f(R, H) for _ in range(L)], [f(R, E) for _ in range(L)]
        self.ti = [torch.empty((R, TOPK), dtype=torch.int32, device="cuda") for _ in range(L)]
        self.z = f(R, V)
        self.toks = torch.empty((1, R), dtype=torch.int32, device="cuda")
        self.nacc = torch.empty((1,), dtype=torch.int32, device="cuda")
        u8 = lambda n: torch.empty(n, dtype=torch.uint8, device="cuda")
        self.ws_moe, self.ws_lm = u8(sv.sv_moe_workspace_bytes(self.desc, R)), u8(sv.sv_lmhead_workspace_bytes(H, R))
        self.ws_acc = u8(sv.sv_accept_workspace_bytes(1, self.K, V))
        self.run(accept=False)
        acc = synth.accept_inputs(host(self.z), 1, self.K, 1.5, 0.8, synth.CFG_LMHEAD, sub=700 + R)
        self.draft = dev(acc.draft_logits) if self.K else None
        self.drafts = dev(acc.drafts) if self.K else None
        self.u = dev(acc.uniforms)

    def run(self, accept=True):
        sv, x = self.sv, self.x
        for l in range(L):
            sv.vq8_lmhead_gemm(self.wr, E, H, x, self.lg[l], ws=self.ws_lm)
            sv.vq2_moe_gemm(self.desc, x, self.lg[l], self.ys[l], self.ti[l], None, ws=self.ws_moe)
            x = self.ys[l]
        sv.vq8_lmhead_gemm(self.wh, V, H, x, self.z, ws=self.ws_lm)
        if accept:
            sv.spec_accept(1, self.K, V, self.z, sv.SV_LOGITS, 0.8, self.draft, sv.SV_LOGITS, 0.8, self.drafts,
                           self.u, self.toks, self.nacc, ws=self.ws_acc)

    def outputs(self):
        return [host(t).copy() for t in self.ys + self.lg + self.ti + [self.z, self.toks, self.nacc]]


@pytest.mark.parametrize("R", [1, 5, 16])
def test_graph_replays_match_eager(sv, model, R):
    import torch
    st = Stack(sv, model, R)
    say("eager step", R)
    st.run()
    want = st.outputs()
    x0 = st.x.clone()
    other = dev(synth.moe_rows(R, synth.CFG_MOE, sub=800 + R).x_bf16)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("capturing the step", R)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work on other inputs first: it overwrites every buffer the graph uses
        st.x.copy_(other)
        st.run()
        torch.cuda.synchronize()
        st.x.copy_(x0)
        torch.cuda.synchronize()
        say("graph replay", rep, "R", R)
        g.replay()
        torch.cuda.synchronize()
        got = st.outputs()
        for i, (a, b) in enumerate(zip(got, want)):
            assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
                f"replay {rep}: output {i} differs from the eager run"
    del g
