#!/usr/bin/env python3
"""Verifier-step benchmark on one MI355X.

One step = the whole verifier hot path on one batch of synthetic input:
  vq2_moe_gemm     one routed MoE layer: 256 two-bit SwiGLU experts + 1 shared
                   (7168 <-> 2048), router top-8, R verifier rows (bf16);
  vq8_lmhead_gemm  the eight-bit vocabulary head 129280 x 7168 on R rows;
  spec_accept      p/q accept/reject with residual resampling for S sequences
                   of K = R/S - 1 drafts at T = 0.8.
Inputs for several batches are generated up front (seeded, synth) and stay
resident in HBM; steps rotate through them.  The timed region is K steps
between two device synchronisations, launched call by call (--launch graph:
each step a replay of a captured HIP graph of the whole step on that batch;
the other mode is timed too and reported beside); value = algorithmic
weight bytes of the timed steps (the routed experts each batch actually
touches, the shared expert, the vocabulary head) / elapsed time.

Prints ONE JSON line (rank 0, N = 1).  Besides the headline (R = 5, S = 1)
the line carries, unless --no-extras: one entry per R = 1..16 and the
three-sequence cohort (R = 15, S = 3), single-expert calls at R = 1, 2, 4, 8
beside an empty-launch floor, live per-kernel times of one R = 5 step with a
roofline entry per expert kernel, the layer with an eight-bit shared expert
and target-sample matching timed beside the step's own calls, the step and a
four-layer stack eagerly and as graph replays, the read-bandwidth probe, and
SHA-256 digests of the generated inputs.  --sweep prints one line per R
instead.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0
Q2_EXPERT_BYTES = 3 * 4816896          # gate + up + down of one 7168 <-> 2048 expert
Q8_HEAD_BYTES = 984596480             # 129280 x 7168 eight-bit blocks


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rows", type=int, default=5, help="verifier rows R (default 5 = 1 + 4 drafts)")
    ap.add_argument("--seqs", type=int, default=1, help="sequences S sharing the rows (R %% S == 0)")
    ap.add_argument("--batches", type=int, default=8, help="distinct input batches rotated over")
    ap.add_argument("--temperature", type=float, default=0.8)
    ap.add_argument("--sweep", default="", help="comma list of R values: one JSON line per R")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=3, help="routed experts in the oracle sample")
    ap.add_argument("--cpu-vocab", type=int, default=16384, help="vocab rows in the oracle sample")
    ap.add_argument("--bw-probe-gib", type=float, default=2.0,
                    help="buffer size of the read-bandwidth probe (0: skip it)")
    ap.add_argument("--bw-probe-only", action="store_true",
                    help="run only the read-bandwidth probe and print its JSON line")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline: no per-R entries, cohort, single-expert calls or kernel times")
    ap.add_argument("--extra-steps", type=int, default=20, help="timed steps of each per-R / cohort entry")
    ap.add_argument("--launch", choices=("eager", "graph"), default="eager",
                    help="timed steps launched call by call (default), or as replays of one captured HIP "
                         "graph per batch; the other mode is timed too and reported beside")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the bench, one plain device copy of this many MiB (fp32 x 1.0): "
                         "the known-size kernel that calibrates profiler byte counters")
    return ap.parse_args()


# ------------------------------------------------------------------ inputs
def gen_moe_weights(threads: int = 8):
    """All 257 experts (seeded per expert), expert-major byte buffers."""
    E = synth.N_ROUTED

    def one(e):
        mats = synth.expert_matrices(synth.CFG_MOE, e)
        return e, [mats[m].packed() for m in (synth.M_GATE, synth.M_UP, synth.M_DOWN)]

    bufs = [None] * (E + 1)
    with cf.ThreadPoolExecutor(threads) as ex:
        for e, b in ex.map(one, range(E + 1)):
            bufs[e] = b
    routed = [np.concatenate([bufs[e][m] for e in range(E)]) for m in range(3)]
    return routed, bufs[E]


def sha256_of(arrays, threads: int = 8) -> str:
    """SHA-256 over the SHA-256 digests of the arrays' bytes, in order (each
    array hashed on its own thread)."""
    def one(a):
        a = np.ascontiguousarray(a)
        return hashlib.sha256(a.tobytes() if a.size == 0 else memoryview(a).cast("B")).digest()
    with cf.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(one, arrays))
    return hashlib.sha256(b"".join(parts)).hexdigest()


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


class Step:
    """Device-resident inputs, outputs and workspaces for one R/S setting."""

    def __init__(self, sv, desc, wq8, R, S, n_batches, temperature):
        import torch
        self.sv, self.desc, self.wq8 = sv, desc, wq8
        self.R, self.S, self.K = R, S, R // S - 1
        self.T = temperature
        V, H = synth.VOCAB, synth.HIDDEN
        self.batches = []
        self.host_inputs = []
        for b in range(n_batches):
            rows = synth.moe_rows(R, synth.CFG_MOE, sub=100 * R + b)
            h = synth.lm_head_hidden(R, synth.CFG_LMHEAD, sub=100 * R + b)
            self.host_inputs += [rows.x_bf16, rows.router_logits, h]
            self.batches.append(dict(x=to_dev(rows.x_bf16), logits=to_dev(rows.router_logits),
                                     h=to_dev(h)))
        self.y = torch.empty((R, H), dtype=torch.float32, device="cuda")
        self.tidx = [torch.empty((R, synth.TOP_K), dtype=torch.int32, device="cuda") for _ in range(n_batches)]
        self.tw = torch.empty((R, synth.TOP_K), dtype=torch.float32, device="cuda")
        self.z = torch.empty((R, V), dtype=torch.float32, device="cuda")
        self.toks = torch.empty((S, self.K + 1), dtype=torch.int32, device="cuda")
        self.nacc = torch.empty((S,), dtype=torch.int32, device="cuda")
        self.ws_moe = torch.empty(sv.sv_moe_workspace_bytes(desc, R), dtype=torch.uint8, device="cuda")
        self.ws_lm = torch.empty(sv.sv_lmhead_workspace_bytes(H, R), dtype=torch.uint8, device="cuda")
        self.ws_acc = torch.empty(sv.sv_accept_workspace_bytes(S, self.K, V), dtype=torch.uint8, device="cuda")
        # draft side: target logits of each batch (one untimed head call), then
        # draft logits = target + N(0, 1.5^2) noise, drafts ~ softmax(draft / T)
        for b, bt in enumerate(self.batches):
            sv.vq8_lmhead_gemm(wq8, V, H, bt["h"], self.z, ws=self.ws_lm)
            torch.cuda.synchronize()
            acc = synth.accept_inputs(self.z.cpu().numpy(), S, self.K, 1.5, temperature,
                                      synth.CFG_LMHEAD, sub=100 * R + b)
            bt["draft"] = to_dev(acc.draft_logits) if self.K else None
            bt["drafts"] = to_dev(acc.drafts) if self.K else None
            bt["u"] = to_dev(acc.uniforms)
            self.host_inputs += [acc.drafts, acc.uniforms] + ([acc.draft_logits] if self.K else [])

    def run(self, b, ev=None):
        sv, bt = self.sv, self.batches[b % len(self.batches)]
        V, H = synth.VOCAB, synth.HIDDEN
        if ev:
            ev[0].record()
        sv.vq2_moe_gemm(self.desc, bt["x"], bt["logits"], self.y, self.tidx[b % len(self.batches)],
                        self.tw, ws=self.ws_moe)
        if ev:
            ev[1].record()
        sv.vq8_lmhead_gemm(self.wq8, V, H, bt["h"], self.z, ws=self.ws_lm)
        if ev:
            ev[2].record()
        sv.spec_accept(self.S, self.K, V, self.z, sv.SV_LOGITS, self.T, bt["draft"], sv.SV_LOGITS,
                       self.T, bt["drafts"], bt["u"], self.toks, self.nacc, ws=self.ws_acc)
        if ev:
            ev[3].record()

    def moe_bytes(self, b):
        """Touched expert bytes of batch b (distinct routed experts + shared)."""
        idx = self.tidx[b % len(self.batches)].cpu().numpy()
        return (len(np.unique(idx)) + 1) * Q2_EXPERT_BYTES


def capture_steps(step):
    """One HIP graph per input batch, each holding one whole step (every
    kernel of the three calls, on that batch's inputs)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for b in range(len(step.batches)):
            step.run(b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for b in range(len(step.batches)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step.run(b)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def measure(step, steps, warmup, launch="eager"):
    """Times `steps` steps with events at the two ends only (an event recorded
    between kernels leaves a gap of several microseconds on the GPU timeline),
    as graph replays (one captured graph per batch) or as eager launches, and
    the other mode the same way for comparison; a further pass over the same
    batches, eager with events around each call, gives the per-call
    breakdown."""
    import torch
    for i in range(warmup):
        step.run(i)
    torch.cuda.synchronize()
    graphs = capture_steps(step)
    nb = len(step.batches)

    def timed(graph):
        # each mode is warmed up by itself first (the first eager steps after
        # a capture run slow)
        for i in range(warmup):
            if graph:
                graphs[i % nb].replay()
            else:
                step.run(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        t0.record()
        for i in range(steps):
            if graph:
                graphs[i % nb].replay()
            else:
                step.run(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1), time.perf_counter() - wall0

    other_ms, _ = timed(launch != "graph")
    total_ms, wall = timed(launch == "graph")
    del graphs
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step.run(i, evs[i])
    torch.cuda.synchronize()
    moe = np.array([e[0].elapsed_time(e[1]) for e in evs])
    lm = np.array([e[1].elapsed_time(e[2]) for e in evs])
    acc = np.array([e[2].elapsed_time(e[3]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    moe_b = np.array([step.moe_bytes(i) for i in range(steps)], np.float64)
    return dict(total_ms=total_ms, wall_s=wall, moe_ms=moe, lm_ms=lm, acc_ms=acc, step_ms=step_ms,
                moe_bytes=moe_b, launch=launch, other_ms=other_ms)


PROBE_MODES = {0: "plain loads to registers, full lines", 1: "global-to-LDS, non-temporal, full lines",
               2: "global-to-LDS, full lines", 3: "global-to-LDS, 64-byte pieces",
               4: "global-to-LDS, non-temporal, 64-byte pieces",
               5: "global-to-LDS 4-byte loads, non-temporal (7 KB of every 28 KB group)"}


def bw_probe(sv, gib: float, reps: int = 10):
    """Read bandwidth of the part with the weight kernels' own load
    instructions (sv_read_probe), each mode timed with HIP events on its launch
    stream over `reps` launches on a buffer far larger than the last-level
    cache: the median GB/s per mode."""
    import torch
    nbytes = int(gib * (1 << 30)) // sv.PROBE_GROUP_BYTES * sv.PROBE_GROUP_BYTES
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    sink = torch.empty(8 * torch.cuda.get_device_properties(0).multi_processor_count, dtype=torch.int32,
                       device="cuda")
    out = {}
    for mode, what in PROBE_MODES.items():
        sv.sv_read_probe(src, mode, sink)   # warm-up
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            nread = sv.sv_read_probe(src, mode, sink)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / 1e3)
        if mode == 5:
            nread = nread // 4   # 7 KB of every 28 KB group
        out[str(mode)] = {"what": what, "GB/s": round(nread / float(np.median(ts)) / 1e9, 1),
                          "us": round(float(np.median(ts)) * 1e6, 1)}
    del src
    torch.cuda.synchronize()
    return {"bytes": nbytes, "modes": out}


# ------------------------------------------------------------------ extras
def entry(R, S, m):
    """Compact per-R record: step time, weight GB/s, roofline fraction and
    the per-call times of the breakdown pass."""
    steps = len(m["step_ms"])
    total_s = m["total_ms"] / 1e3
    gbs = float((m["moe_bytes"] + Q8_HEAD_BYTES).sum() / total_s / 1e9)
    other = "eager" if m["launch"] == "graph" else "graph"
    return {"R": R, "S": S, "K": R // S - 1, "ms_per_step": round(total_s * 1e3 / steps, 4),
            f"{other}_ms_per_step": round(m["other_ms"] / steps, 4),
            "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "call_us": {"vq2_moe_gemm": round(float(m["moe_ms"].mean()) * 1e3, 2),
                        "vq8_lmhead_gemm": round(float(m["lm_ms"].mean()) * 1e3, 2),
                        "spec_accept": round(float(m["acc_ms"].mean()) * 1e3, 2)},
            "moe_GB/s": round(float(m["moe_bytes"].sum() / (m["moe_ms"].sum() / 1e3) / 1e9), 1)}


def single_expert(sv, desc, Rs=(1, 2, 4, 8), copies: int = 24):
    """Config C1 shape: one SwiGLU expert (E = 1, no shared) with all R rows.
    One timed unit is `copies` calls back to back, each on its own resident
    expert (24 x 14.45 MB exceeds the 256 MB last-level cache, so the weights
    stream from HBM), run eagerly and as a captured graph; the per-call time is
    the unit's median over the copies.  Eager calls of this size are bound by
    the host's launch rate, so `frac` is taken from the graph replay.  Beside
    it, the time of five minimal kernels (one-element fills), the floor of any
    five-launch call, timed the same way."""
    import torch
    wg, wu, wd = desc._keep[0], desc._keep[1], desc._keep[2]
    gu, dn = sv.sv_q2_tiled_bytes(synth.INTER, synth.HIDDEN), sv.sv_q2_tiled_bytes(synth.HIDDEN, synth.INTER)
    descs = [sv.moe_desc(sv.SV_FFN_SWIGLU, synth.HIDDEN, synth.INTER, 1, 1, wg[e * gu:(e + 1) * gu],
                         wu[e * gu:(e + 1) * gu], wd[e * dn:(e + 1) * dn], tiled=True)
             for e in range(copies)]
    t = torch.empty(1, dtype=torch.float32, device="cuda")

    def empties():
        for _ in range(5 * copies):
            t.fill_(1.0)

    floor_e, floor_g = time_eager_and_graph(empties, reps=12)
    out = []
    for R in Rs:
        x = to_dev(synth.expert(R).x_bf16)
        y = torch.empty((R, synth.HIDDEN), dtype=torch.float32, device="cuda")
        ws = torch.empty(sv.sv_moe_workspace_bytes(descs[0], R), dtype=torch.uint8, device="cuda")

        def unit():
            for d in descs:
                sv.vq2_moe_gemm(d, x, None, y, ws=ws)

        eager, graph = time_eager_and_graph(unit, reps=12)
        us_e, us_g = eager / copies, graph / copies
        out.append({"R": R, "us_eager": round(us_e, 2), "us": round(us_g, 2),
                    "GB/s": round(Q2_EXPERT_BYTES / us_g / 1e3, 1),
                    "frac": round(Q2_EXPERT_BYTES / us_g / 1e3 / PEAK_HBM_GBS, 4)})
        del ws, x, y
        torch.cuda.synchronize()
    return {"bytes": Q2_EXPERT_BYTES, "launches": 5, "calls_per_unit": copies,
            "empty_launch_floor_us": {"eager": round(floor_e / copies, 2), "graph": round(floor_g / copies, 2)},
            "rows": out}


def event_median(call, reps: int = 40) -> float:
    """Median event-timed duration of call() in microseconds."""
    import torch
    call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts)) * 1e3


def next_rows(sv, step, wroute):
    """The rows beyond the verifier step proper, timed at the step's shape:
    the layer with its shared expert in eight-bit blocks beside the two-bit
    one (the same routed experts and rows), and target-sample matching beside
    the p/q rule on the step's own logits."""
    import torch
    wg, wu, wd = wroute
    sq = [to_dev(m.packed()) for m in synth.shared_q8_weights()]
    d8 = sv.moe_desc(sv.SV_FFN_SWIGLU, synth.HIDDEN, synth.INTER, synth.N_ROUTED, synth.TOP_K, wg, wu, wd,
                     *sq, tiled=True, shared_format=sv.SV_Q8)
    ws8 = torch.empty(sv.sv_moe_workspace_bytes(d8, step.R), dtype=torch.uint8, device="cuda")
    bt = step.batches[0]
    q2 = event_median(lambda: sv.vq2_moe_gemm(step.desc, bt["x"], bt["logits"], step.y, ws=step.ws_moe))
    q8 = event_median(lambda: sv.vq2_moe_gemm(d8, bt["x"], bt["logits"], step.y, ws=ws8))
    q8_bytes = 2 * sv.sv_q8_matrix_bytes(synth.INTER, synth.HIDDEN) + sv.sv_q8_matrix_bytes(synth.HIDDEN, synth.INTER)
    V = synth.VOCAB
    sv.vq8_lmhead_gemm(step.wq8, V, synth.HIDDEN, bt["h"], step.z, ws=step.ws_lm)
    ws_t = torch.empty(sv.sv_accept_tsm_workspace_bytes(step.S, step.K, V), dtype=torch.uint8, device="cuda")
    pq = event_median(lambda: sv.spec_accept(step.S, step.K, V, step.z, sv.SV_LOGITS, step.T, bt["draft"],
                                             sv.SV_LOGITS, step.T, bt["drafts"], bt["u"], step.toks, step.nacc,
                                             ws=step.ws_acc))
    ts = event_median(lambda: sv.spec_accept_target_sample(step.S, step.K, V, step.z, sv.SV_LOGITS, step.T,
                                                           bt["drafts"], bt["u"], step.toks, step.nacc, ws=ws_t))
    return {"R": step.R, "S": step.S, "K": step.K,
            "moe_layer_us": {"shared_q2": round(q2, 2), "shared_q8": round(q8, 2)},
            "shared_expert_bytes": {"q2": Q2_EXPERT_BYTES, "q8": q8_bytes},
            "accept_us": {"p_q_rule": round(pq, 2), "target_sample_matching": round(ts, 2)}}


KERNEL_KEYS = {"gate/up": "k_gu8", "down": "k_dn8", "down input digits": "k_hdig", "routing": "k_moe_prep",
               "combine": "k_moe_combine", "head": "k_q8_lmhead", "head staging": "k_stage",
               "accept statistics": "k_acc_stats", "accept sample": "k_acc_sample", "accept pick": "k_acc_pick",
               "target-sample matching": "k_tsm_pick", "shared expert h staging": "k_stage_swiglu"}


def kernel_times(step, steps: int = 10):
    """Average device time per launch of each kernel over `steps` steps,
    from torch's profiler (it records the library's launches on the same
    stream); with the algorithmic bytes of the two expert kernels, their
    roofline entries.  None when the profiler is unavailable."""
    import torch
    try:
        from torch.profiler import ProfilerActivity, profile
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for i in range(steps):
                step.run(i)
            torch.cuda.synchronize()
        avg = {}
        for ev in prof.key_averages():
            dev_us = getattr(ev, "device_time_total", None)
            if dev_us is None:
                dev_us = getattr(ev, "cuda_time_total", 0.0)
            if ev.count and dev_us:
                for what, key in KERNEL_KEYS.items():
                    if key in ev.key:
                        a = avg.setdefault(what, {"kernel": ev.key.split("(")[0].replace("void ", ""),
                                                  "launches": 0, "us_total": 0.0})
                        a["launches"] += ev.count
                        a["us_total"] += dev_us
    except Exception as exc:  # pragma: no cover - profiler support differs between builds
        log(f"kernel times unavailable: {exc!r}")
        return None
    out = {}
    for what, a in avg.items():
        out[what] = {"kernel": a["kernel"], "launches": a["launches"],
                     "us": round(a["us_total"] / a["launches"], 2)}
    # algorithmic bytes per launch of the expert kernels: each touched expert's
    # matrices once (gate + up for the first, down for the second)
    per = Q2_EXPERT_BYTES // 3
    experts = float(np.mean([len(np.unique(step.tidx[i % len(step.batches)].cpu().numpy())) + 1
                             for i in range(steps)]))
    roof = []
    for what, nbytes in (("gate/up", 2 * per * experts), ("down", per * experts)):
        if what in out:
            gbs = nbytes / (out[what]["us"] * 1e-6) / 1e9
            roof.append({"kernel": out[what]["kernel"], "bound": "hbm", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "bytes_per_launch": int(nbytes)})
    return {"steps": steps, "R": step.R, "kernels": out, "roofline_expert_kernels": roof}


class LayerStack:
    """A verifier step over L stacked MoE layers: per layer the eight-bit
    router GEMV ([256 x 7168], through the head's call) on the layer's input,
    the routed layer, its output feeding the next layer (fp32); then the
    vocabulary head on the last output and spec_accept (S = 1, K = R - 1).
    The layers share one expert set and router (a synthetic stand-in: the
    work per layer is the same as with distinct weights, the touched experts
    differ with the inputs)."""

    def __init__(self, sv, desc, wq8, wrouter, R, L, temperature):
        import torch
        self.sv, self.desc, self.wq8, self.wr = sv, desc, wq8, wrouter
        self.R, self.L, self.K, self.T = R, L, R - 1, temperature
        V, H, E = synth.VOCAB, synth.HIDDEN, synth.N_ROUTED
        self.x0 = to_dev(synth.moe_rows(R, synth.CFG_MOE, sub=900 + R).x_bf16)
        self.ys = [torch.empty((R, H), dtype=torch.float32, device="cuda") for _ in range(L)]
        self.lg = [torch.empty((R, E), dtype=torch.float32, device="cuda") for _ in range(L)]
        self.tidx = torch.empty((R, synth.TOP_K), dtype=torch.int32, device="cuda")
        self.z = torch.empty((R, V), dtype=torch.float32, device="cuda")
        self.toks = torch.empty((1, R), dtype=torch.int32, device="cuda")
        self.nacc = torch.empty((1,), dtype=torch.int32, device="cuda")
        self.ws_moe = torch.empty(sv.sv_moe_workspace_bytes(desc, R), dtype=torch.uint8, device="cuda")
        self.ws_lm = torch.empty(sv.sv_lmhead_workspace_bytes(H, R), dtype=torch.uint8, device="cuda")
        self.ws_acc = torch.empty(sv.sv_accept_workspace_bytes(1, self.K, V), dtype=torch.uint8, device="cuda")
        self.draft = self.drafts = None
        self.u = torch.zeros((1, R), dtype=torch.float32, device="cuda")
        self.run()                       # target logits of the stack, then the draft side
        torch.cuda.synchronize()
        acc = synth.accept_inputs(self.z.cpu().numpy(), 1, self.K, 1.5, temperature, synth.CFG_LMHEAD, sub=900 + R)
        self.draft = to_dev(acc.draft_logits) if self.K else None
        self.drafts = to_dev(acc.drafts) if self.K else None
        self.u = to_dev(acc.uniforms)

    launches_per_layer = 2 + 5          # router GEMV (staging + head kernel) + the MoE layer

    def launches(self):
        return self.L * self.launches_per_layer + 2 + 2

    def run(self):
        sv, H, V, E = self.sv, synth.HIDDEN, synth.VOCAB, synth.N_ROUTED
        x = self.x0
        for l in range(self.L):
            sv.vq8_lmhead_gemm(self.wr, E, H, x, self.lg[l], ws=self.ws_lm)
            sv.vq2_moe_gemm(self.desc, x, self.lg[l], self.ys[l], self.tidx, None, ws=self.ws_moe)
            x = self.ys[l]
        sv.vq8_lmhead_gemm(self.wq8, V, H, x, self.z, ws=self.ws_lm)
        if self.u is not None and (self.K == 0 or self.draft is not None):
            sv.spec_accept(1, self.K, V, self.z, sv.SV_LOGITS, self.T, self.draft, sv.SV_LOGITS, self.T,
                           self.drafts, self.u, self.toks, self.nacc, ws=self.ws_acc)


def time_eager_and_graph(fn, reps: int = 30):
    """Median event-timed duration of fn() run eagerly and as a captured HIP
    graph replay (torch.cuda.CUDAGraph), in microseconds."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()

    def timed(call):
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)) * 1e3

    eager = timed(fn)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    graph = timed(g.replay)
    del g
    return eager, graph


def graph_steps(sv, desc, wq8, Rs=(1, 5, 16), L: int = 4):
    """The verifier step (one MoE layer + head + accept) and an L-layer step
    (router GEMV + MoE per layer, then head + accept), each timed eagerly and
    as a graph replay at every R."""
    import torch
    wr = to_dev(synth.router_weights().packed())
    out = []
    for R in Rs:
        st = Step(sv, desc, wq8, R, 1, 1, 0.8)
        e1, g1 = time_eager_and_graph(lambda: st.run(0))
        del st
        stack = LayerStack(sv, desc, wq8, wr, R, L, 0.8)
        eL, gL = time_eager_and_graph(stack.run)
        out.append({"R": R, "step_us": {"eager": round(e1, 2), "graph": round(g1, 2)},
                    f"stack{L}_us": {"eager": round(eL, 2), "graph": round(gL, 2),
                                     "launches": stack.launches()}})
        del stack
        torch.cuda.synchronize()
    return {"layers": L, "rows": out}


def cpu_baseline(step_bytes_mean, R, n_experts, n_vocab):
    """The oracle, unchanged, on a bounded sample of the same workload."""
    import threadpoolctl
    import oracle
    x_rows = synth.moe_rows(R, synth.CFG_MOE, sub=100 * R)
    idx, _ = oracle.route_topk(x_rows.router_logits, synth.TOP_K)
    experts = sorted(set(idx.reshape(-1).tolist()))[:n_experts]
    x64 = oracle.linalg._exact_rows(x_rows.x_bf16, "bf16")
    mats = {e: synth.expert_matrices(synth.CFG_MOE, e) for e in experts + [synth.N_ROUTED]}
    packed = {e: [mats[e][m].packed() for m in range(3)] for e in mats}
    q8 = synth.q8_random(synth.generator(synth.CFG_LMHEAD, synth.S_WEIGHTS), n_vocab, synth.HIDDEN, 0.01).packed()
    h = synth.lm_head_hidden(R, synth.CFG_LMHEAD, sub=100 * R)
    # warm the BLAS pool (untimed)
    oracle.swiglu_expert(*packed[experts[0]], synth.HIDDEN, synth.INTER, x64[:1])
    t0 = time.perf_counter()
    for e in experts:
        rows = sorted(set(np.nonzero(idx == e)[0].tolist()))
        oracle.swiglu_expert(*packed[e], synth.HIDDEN, synth.INTER, x64[rows])
    oracle.swiglu_expert(*packed[synth.N_ROUTED], synth.HIDDEN, synth.INTER, x64)
    z = oracle.lm_head_logits(q8, n_vocab, synth.HIDDEN, h, "bf16")
    S, K = 1, R - 1
    tl = z.astype(np.float32)
    acc_in = synth.accept_inputs(tl, S, K, 1.5, 0.8, synth.CFG_LMHEAD, sub=0)
    oracle.spec_accept(S, K, n_vocab, tl, 0, 0.8, acc_in.draft_logits, 0, 0.8, acc_in.drafts,
                       acc_in.uniforms)
    dt = time.perf_counter() - t0
    nbytes = (len(experts) + 1) * Q2_EXPERT_BYTES + n_vocab * synth.HIDDEN * 34 // 32
    threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    model = platform.processor() or platform.machine()
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    gbs = nbytes / dt / 1e9
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{len(experts)} routed experts (their routed rows) + the shared expert on "
                       f"{R} rows, vocabulary head over {n_vocab} of {synth.VOCAB} rows, and "
                       f"spec_accept (S=1, K={K}) over those {n_vocab} logits; {nbytes / 1e6:.1f} MB "
                       f"of weights in {dt:.2f} s"),
            "seconds": round(dt, 3),
            "est_step_s": round(step_bytes_mean / (gbs * 1e9), 2),
            "cpu": model, "host_cpus": os.cpu_count(),
            "threads_note": "cores = threads of the BLAS pool the oracle's matrix products ran on"}


TRAFFIC_PROFILE = os.path.join(HERE, "profiles", "verifier_step_R5_hbm_traffic.md")


def head_traffic(R):
    """HBM bytes per vq8_lmhead_gemm call from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the copy-kernel
    calibration), or None: for another R, or once a source the counters were
    taken on has changed."""
    import hashlib
    if R != 5 or not os.path.exists(TRAFFIC_PROFILE):
        return None
    text = open(TRAFFIC_PROFILE).read()
    a = text.find("```json")
    if a < 0:
        return None
    b = text.find("```", a + 7)
    data = json.loads(text[a + 7:b])
    for name, digest in data["sources_sha256"].items():
        path = os.path.join(HERE, "bit_moe_tiny_amd", "csrc", name)
        if not os.path.exists(path) or hashlib.sha256(open(path, "rb").read()).hexdigest() != digest:
            return None
    kib = sum(k["fetch_kib"] * data["fetch_factor"] + k["write_kib"] * data["write_factor"]
              for k in data["kernels"].values())
    return int(round(kib * 1024))


def result_line(args, R, S, m, cpu=None):
    steps = len(m["step_ms"])
    total_s = m["total_ms"] / 1e3
    head_act = R * synth.HIDDEN * 2 + R * synth.VOCAB * 4
    step_bytes = m["moe_bytes"] + Q8_HEAD_BYTES
    gbs = float(step_bytes.sum() / total_s / 1e9)
    lm_ms = float(m["lm_ms"].mean())
    lm_bytes = Q8_HEAD_BYTES + head_act
    achieved = lm_bytes / (lm_ms / 1e3) / 1e9
    line = {
        "metric": "verifier-step µs and weight HBM GB/s (Q2 MoE + Q8 lm_head, R=1..16)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_s * 1e3 / steps, 4),
        "launch": m["launch"],
        ("eager" if m["launch"] == "graph" else "graph") + "_ms_per_step": round(m["other_ms"] / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"verifier step: MoE layer (256 routed + 1 shared two-bit SwiGLU experts, "
                         f"7168<->2048, top-8) + eight-bit vocabulary head 129280x7168 + "
                         f"spec_accept, R={R} rows, S={S} sequence(s) x K={R // S - 1} drafts, T=0.8"),
            "R": R, "S": S, "K": R // S - 1, "batches": args.batches,
        },
        # per-step spread and per-call times: the breakdown pass (events
        # between the calls add their own gaps, so these exceed ms_per_step)
        "step_us": {"median": round(float(np.median(m["step_ms"])) * 1e3, 2),
                    "p10": round(float(np.percentile(m["step_ms"], 10)) * 1e3, 2),
                    "p90": round(float(np.percentile(m["step_ms"], 90)) * 1e3, 2)},
        "call_us": {"vq2_moe_gemm": round(float(m["moe_ms"].mean()) * 1e3, 2),
                    "vq8_lmhead_gemm": round(lm_ms * 1e3, 2),
                    "spec_accept": round(float(m["acc_ms"].mean()) * 1e3, 2)},
        "weight_bytes_per_step": int(step_bytes.mean()),
        "moe_gbs": round(float(m["moe_bytes"].sum() / (m["moe_ms"].sum() / 1e3) / 1e9), 1),
        "hbm_frac_step": round(gbs / PEAK_HBM_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": head_traffic(R),
                     "kernel": "vq8_lmhead_gemm (one call: k_stage + k_q8_lmhead_dma)",
                     "bytes_per_launch": lm_bytes},
        "wall_s": round(m["wall_s"], 3),
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the verifier step "
              "is measured per GPU and nothing here spans several GPUs.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_moe_tiny_amd as sv
    sv.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.bw_probe_only:
        log(f"read-bandwidth probe on {args.bw_probe_gib} GiB")
        print(json.dumps({"bw_probe": bw_probe(sv, args.bw_probe_gib)}), flush=True)
        return
    t = time.time()
    log("generating 257 two-bit experts (3.7 GB) ...")
    (g, u, d), (sg, su, sd) = gen_moe_weights()
    digests = {"moe_weights": sha256_of([g, u, d, sg, su, sd])}
    wg, wu, wd, wsg, wsu, wsd = (to_dev(a) for a in (g, u, d, sg, su, sd))
    del g, u, d
    log(f"experts resident ({time.time() - t:.1f} s); generating the vocabulary head (985 MB) ...")
    q8 = synth.lm_head_weights().packed()
    digests["head_weights"] = sha256_of([q8])
    wq8 = to_dev(q8)
    del q8
    log(f"head resident ({time.time() - t:.1f} s)")
    desc = sv.moe_desc(sv.SV_FFN_SWIGLU, synth.HIDDEN, synth.INTER, synth.N_ROUTED, synth.TOP_K,
                       wg, wu, wd, wsg, wsu, wsd)
    rs = [int(r) for r in args.sweep.split(",")] if args.sweep else [args.rows]
    for R in rs:
        S = args.seqs if R % args.seqs == 0 else 1
        step = Step(sv, desc, wq8, R, S, args.batches, args.temperature)
        log(f"R={R} S={S}: {args.warmup} warmup + {args.steps} timed steps")
        m = measure(step, args.steps, args.warmup, args.launch)
        cpu = None
        if not args.no_cpu_baseline and not args.sweep:
            log("cpu_baseline: timing the oracle on a bounded sample ...")
            cpu = cpu_baseline(float((m["moe_bytes"] + Q8_HEAD_BYTES).mean()), R, args.cpu_experts,
                               args.cpu_vocab)
        line = result_line(args, R, S, m, cpu)
        if not args.sweep:
            digests["step_inputs"] = sha256_of(step.host_inputs)
            line["inputs_sha256"] = digests
            if not args.no_extras:
                log("kernel times of one step (profiler) ...")
                line["kernel_times"] = kernel_times(step)
                log("eight-bit shared expert and target-sample matching ...")
                line["next_rows"] = next_rows(sv, step, (desc._keep[0], desc._keep[1], desc._keep[2]))
                del step
                ents = []
                for r2, s2 in [(r, 1) for r in range(1, 17)] + [(15, 3)]:
                    st = Step(sv, desc, wq8, r2, s2, 3, args.temperature)
                    ents.append(entry(r2, s2, measure(st, args.extra_steps, 3, args.launch)))
                    log(f"entry R={r2} S={s2}: {ents[-1]['ms_per_step']} ms per step")
                    del st
                line["per_R"] = [e for e in ents if e["S"] == 1]
                line["cohort"] = [e for e in ents if e["S"] == 3][0]
                log("single-expert calls ...")
                line["single_expert"] = single_expert(sv, desc)
                log("eager and graph-replayed steps ...")
                line["graph_steps"] = graph_steps(sv, desc, wq8)
            if args.bw_probe_gib > 0:
                log(f"read-bandwidth probe on {args.bw_probe_gib} GiB ...")
                line["bw_probe"] = bw_probe(sv, args.bw_probe_gib)
        print(json.dumps(line), flush=True)
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")


if __name__ == "__main__":
    main()
