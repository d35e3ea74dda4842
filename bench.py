#!/usr/bin/env python3
"""Benchmark of the BitNet b1.58 BitLinear forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]

Headline (``value``): prefill throughput of a 700M LLaMA-shape layer
(hidden 1536, FFN 4096, 2048 tokens), one step = the per-token activation
quantisation of the layer's four inputs plus its seven BitLinear forwards
(Q, K, V, O, gate, up, down) issued as a serving engine does, in the groups
that share an input (QKV grouped, O, gate+up grouped, down), in int8 TOPS
(2*M*N*K ops per forward).  The decode half of the metric (``decode`` and
the ``decode_*`` fields) is the 70B LLaMA-shape layer (hidden 8192, FFN
28672, GQA K/V 1024) at 1, 16 and 64 tokens and the 3B layer at 1 and 8
tokens: per input, its activation quant and the forwards that read it in one
call, in GB/s of algorithmic bytes.  Also measured: the single BitLinear
256 -> 512 at 32 tokens (absolute us), the 42 forwards of the 6-layer model
at 8192 tokens (GB/s), the weight packer and the sign-flip tracker, the
RMSNorm + quant, the straight-through backward, the fused AdamW + tracker,
the measured HBM / int8 MFMA peaks of the GPU (bench_peaks.hip), and the CPU
oracle step by step.  The summary line stays small; every measurement goes
to stderr (``# detail``) and, with --detail-out, to a file.

Inputs are seeded synthetic tensors (workloads/), resident in HBM before the
timed region.  Steps are replayed from HIP graphs, as a serving loop runs
them: one graph holds a cycle of steps through the rotation sets of buffers
(so the 256 MB last-level cache cannot hold the working set), replayed
whole, and single-step graphs make up a remainder of --steps; per-kernel
durations come from HIP events around graph replays of that kernel alone on
the stream it runs on.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "BitLinear TOPS (prefill, % int8 MFMA peak) + decode GEMV GB/s (% HBM peak)"
PEAK_INT8_TOPS = 5000.0   # MI355X dense int8 MFMA, 5.0 POP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 << 20
PROJ = ["q", "k", "v", "o", "gate", "up", "down"]
INPUTS = ["qkv", "o", "gateup", "down"]


def fwd_bytes(M, N, K):
    """Algorithmic bytes of one forward: 2-bit codes + int8 x + scales + gamma + bf16 y."""
    return N * K // 4 + M * K + 4 * M + 4 + 2 * M * N


def fwd_ops(M, N, K):
    return 2 * M * N * K


def fwd_bytes_b1(M, N, K):
    """Algorithmic bytes of one forward over layout b1: 1-bit codes + int8 x + scales + beta + bf16 y."""
    return N * K // 8 + M * K + 4 * M + 4 + 2 * M * N


def quant_bytes(M, K):
    return 3 * M * K + 4 * M


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--quick", action="store_true", help="prefill only (for profiling runs)")
    ap.add_argument("--only", choices=["prefill", "decode", "aux", "small", "peaks", "b1"], default=None)
    ap.add_argument("--b1", default="70B:1,16;3B:1",
                    help="decode workloads of the one-bit binary layout (as --decode)")
    ap.add_argument("--detail-out", default=None, help="also write every measurement to this JSON file")
    ap.add_argument("--eager-only", choices=["all", "prefill", "decode", "forwards", "batch"], default="all",
                    help="with --eager-kernels: which launches to make")
    ap.add_argument("--decode", default="70B:1,16,64;3B:1,8",
                    help="decode workloads, e.g. '70B:1' (layer:token counts; layers 70B, 3B)")
    ap.add_argument("--no-per-proj", action="store_true",
                    help="skip the per-projection kernel timings (profiling runs)")
    ap.add_argument("--eager-kernels", type=int, default=0, metavar="R",
                    help="no timing: launch a reference copy, the prefill forwards and the 70B M=1 decode "
                         "forwards R times each without graphs (for hardware-counter runs), then exit")
    return ap.parse_args()


class Weights:
    """Packed weights of one LLaMA-shape layer, `sets` independent copies
    (b1: binary weights in the one-bit layout, (packed, beta) per tensor)."""

    def __init__(self, bl, torch, wl, name, sets, layer=0, b1=False):
        shapes = wl.WORKLOADS[name]["tensors"]
        self.shapes = shapes
        self.layer = layer
        base = {}
        for p in PROJ:
            W = torch.from_numpy(wl.workload_weight(name, p, layer)).cuda()
            base[p] = bl.pack_binary_b1(W)[:2] if b1 else bl.pack_weights(W)
            del W
        self.sets = [base] + [{p: (base[p][0].clone(), base[p][1].clone()) for p in PROJ} for _ in range(sets - 1)]

    def bytes(self):
        return sum(self.sets[0][p][0].numel() for p in PROJ)


class Layer:
    """Activation buffers of one LLaMA-shape layer at M tokens over a set of
    packed weight copies (rotated through to defeat the last-level cache)."""

    def __init__(self, bl, torch, wl, name, M, weights):
        self.bl, self.torch, self.name, self.M = bl, torch, name, M
        shapes = wl.WORKLOADS[name]["tensors"]
        self.shapes = shapes
        self.w = weights.sets
        sets = len(self.w)
        kin = {"qkv": shapes["q"][1], "o": shapes["o"][1], "gateup": shapes["gate"][1], "down": shapes["down"][1]}
        rep = {"qkv": "q", "o": "o", "gateup": "gate", "down": "down"}
        base_x = {i: torch.from_numpy(wl.workload_activation(name, rep[i], M, weights.layer).view(np.int16)).cuda()
                  .view(torch.bfloat16) for i in INPUTS}
        self.x, self.q, self.y = [], [], []
        for s in range(sets):
            self.x.append({i: base_x[i].clone() for i in INPUTS})
            self.q.append({i: (torch.empty((M, kin[i]), dtype=torch.int8, device="cuda"),
                               torch.empty(M, dtype=torch.float32, device="cuda")) for i in INPUTS})
            self.y.append({p: torch.empty((M, shapes[p][0]), dtype=torch.bfloat16, device="cuda") for p in PROJ})
        self.kin = kin
        self.input_of = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup", "up": "gateup",
                         "down": "down"}

    def quant(self, s):
        for i in INPUTS:
            self.bl.quant_act(self.x[s][i], xq=self.q[s][i][0], x_scale=self.q[s][i][1])

    def forward(self, s, p):
        N, K = self.shapes[p]
        xq, xs = self.q[s][self.input_of[p]]
        packed, g = self.w[s][p]
        self.bl.forward(packed, g, N, K, xq, xs, y=self.y[s][p])

    def step(self, s):
        """Prefill step in the order a layer runs it: each input's activation
        quant right before the forwards that read it, the seven forwards
        grouped the way they share inputs (QKV, O, gate+up, down)."""
        xq = self.q[s]
        for i, ps in (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",))):
            self.bl.quant_act(self.x[s][i], xq=xq[i][0], x_scale=xq[i][1])
            if len(ps) > 1:
                self.bl.forward_grouped([self.entry(s, p) for p in ps])
            else:
                self.forward(s, ps[0])

    def entry(self, s, p):
        N, K = self.shapes[p]
        xq, xs = self.q[s][self.input_of[p]]
        packed, g = self.w[s][p]
        return dict(packed=packed, gamma=g, N=N, K=K, xq=xq, x_scale=xs, y=self.y[s][p])

    def forward_fused(self, s):
        """The layer's seven forwards as a serving engine runs them: Q, K, V in
        one grouped call (they read the same tokens), O, gate and up in one
        grouped call, down.  The same calls serve prefill and decode; the
        library picks the kernels by token count."""
        self.bl.forward_grouped([self.entry(s, p) for p in ("q", "k", "v")])
        self.forward(s, "o")
        self.bl.forward_grouped([self.entry(s, p) for p in ("gate", "up")])
        self.forward(s, "down")

    GROUPS = (("qkv", ("q", "k", "v")), ("o", ("o",)), ("gateup", ("gate", "up")), ("down", ("down",)))

    def qentry(self, s, p):
        N, K = self.shapes[p]
        i = self.input_of[p]
        packed, g = self.w[s][p]
        xq, xs = self.q[s][i]
        return dict(packed=packed, gamma=g, N=N, K=K, x=self.x[s][i], xq=xq, x_scale=xs, y=self.y[s][p])

    def decode_step(self, s):
        """Decode step as a serving loop runs it: per input, its activation
        quant and the forwards that read it in one call (one launch when the
        tokens are few enough for the decode kernel to quantise them itself)."""
        for _, ps in self.GROUPS:
            self.bl.quant_forward_grouped([self.qentry(s, p) for p in ps])

    def step_bytes(self):
        """Algorithmic bytes of one step: codes, bf16 y, gamma per forward; bf16
        x read and int8 codes + fp32 scales written per input."""
        M = self.M
        b = sum(self.shapes[p][0] * self.shapes[p][1] // 4 + 2 * M * self.shapes[p][0] + 4 for p in PROJ)
        return b + sum(3 * M * self.kin[i] + 4 * M for i in INPUTS)

    def fused_launches(self):
        """Launches of decode_step: one per input where the decode kernel
        quantises the tokens itself (one token with K <= 32768, or 2..16
        tokens with M*K <= 16384), else two."""
        def one(K):
            return K <= 32768 if self.M == 1 else self.M <= 16 and self.M * K <= 16384
        return sum(1 if one(self.kin[i]) else 2 for i in INPUTS)

    def ops(self):
        return sum(fwd_ops(self.M, *self.shapes[p]) for p in PROJ)


def rotation_sets(per_set_bytes):
    """Copies needed so that one pass over all of them exceeds twice the MALL."""
    return max(2, int(np.ceil(2 * MALL_BYTES / per_set_bytes)))


def capture(torch, fn, sets):
    """One HIP graph per rotation set."""
    graphs = []
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for s in range(sets):
            fn(s)  # warm (first call caches the device check)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for s in range(sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(s)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_cycle(torch, fn, sets):
    """A serving loop's graphs: one graph holding a whole cycle of steps
    through the rotation sets (step s on set s), so the host launches one
    graph per cycle instead of one per step, and one single-step graph per
    set for a remainder."""
    singles = capture(torch, fn, sets)
    cycle = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cycle):
        for s in range(sets):
            fn(s)
    torch.cuda.synchronize()
    return cycle, singles


def replay_steps(torch, cycle, singles, steps, warmup):
    """Exactly `steps` steps (whole cycles, then single steps), after
    `warmup` steps, bracketed by synchronize; returns (wall seconds, event
    milliseconds)."""
    sets = len(singles)

    def run(n):
        for _ in range(n // sets):
            cycle.replay()
        for i in range(n % sets):
            singles[i].replay()

    run(warmup)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    run(steps)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, e0.elapsed_time(e1)


def replay_timed(torch, graphs, steps, warmup):
    """Warm-up replays, then exactly `steps` replays bracketed by synchronize;
    returns (wall seconds, event milliseconds)."""
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, e0.elapsed_time(e1)


def kernel_avg_us(torch, layer, fn_per_set, launches_per_call, reps):
    """Average duration of one launch, from HIP events around replays of a
    graph that holds only that kernel's launches, cycling through the
    rotation sets (several launches per replay keep the GPU queue full)."""
    sets = len(layer.w)
    per_graph = sets * max(1, 16 // sets)

    def body(_s):
        for i in range(per_graph):
            fn_per_set(i % sets)

    graphs = capture(torch, body, 1)
    n = max(2, reps // per_graph)
    _, ms = replay_timed(torch, graphs, n, 2)
    return ms * 1e3 / (n * per_graph * launches_per_call)


def bench_prefill(bl, torch, wl, steps, warmup, per_proj=True):
    M = 2048
    probe = wl.WORKLOADS["layer_700m"]["tensors"]
    per_set = sum(fwd_bytes(M, *probe[p]) for p in PROJ)
    sets = rotation_sets(per_set)
    layer = Layer(bl, torch, wl, "layer_700m", M, Weights(bl, torch, wl, "layer_700m", sets))
    cycle, graphs = capture_cycle(torch, layer.step, sets)
    wall, ev_ms = replay_steps(torch, cycle, graphs, steps, warmup)
    ms_step = 1e3 * wall / steps
    ops = layer.ops()
    out = {"ms_per_step": ms_step, "event_ms_per_step": ev_ms / steps, "ops_per_step": ops,
           "tops": ops / (ms_step * 1e-3) / 1e12, "rotation_sets": sets}
    tot_ops = sum(fwd_ops(M, *layer.shapes[p]) for p in PROJ)
    if per_proj:  # each forward as a launch of its own, for reference
        per = {}
        tot_us = 0.0
        for p in PROJ:
            us = kernel_avg_us(torch, layer, lambda s, p=p: layer.forward(s, p), 1, max(steps, 20))
            N, K = layer.shapes[p]
            per[p] = {"N": N, "K": K, "us": us, "tops": fwd_ops(M, N, K) / (us * 1e-6) / 1e12}
            tot_us += us
        out["per_projection"] = per
        out["separate_us_sum"] = tot_us
        out["separate_tops"] = tot_ops / (tot_us * 1e-6) / 1e12
    qus = kernel_avg_us(torch, layer, layer.quant, len(INPUTS), max(steps, 20))
    # the step's four GEMM launches (QKV grouped, O, gate+up grouped, down)
    fused_us = kernel_avg_us(torch, layer, layer.forward_fused, 1, max(steps, 20))
    out["gemm_us_sum"] = fused_us
    out["gemm_tops"] = tot_ops / (fused_us * 1e-6) / 1e12
    out["quant_us_avg"] = qus
    out["quant_gbs"] = sum(quant_bytes(M, layer.kin[i]) for i in INPUTS) / (qus * len(INPUTS) * 1e-6) / 1e9
    out["gemm_ops_per_launch_avg"] = tot_ops / 4
    out["gemm_us_per_launch_avg"] = fused_us / 4
    del layer, graphs, cycle
    torch.cuda.empty_cache()
    return out


def bench_decode(bl, torch, wl, wname, Ms, steps, warmup, per_proj=True):
    """One decode step = per input, the activation quant and the forwards that
    read it (QKV grouped, O, gate+up grouped, down) as one call each
    (bitlinear_quant_forward_grouped).  Also timed: the same forwards alone
    on quantised inputs (4 launches), and the step with separate quant
    launches (8 launches)."""
    res = {}
    shapes = wl.WORKLOADS[wname]["tensors"]
    packed_bytes = sum(bl.packed_bytes(*shapes[p]) for p in PROJ)
    weights = Weights(bl, torch, wl, wname, rotation_sets(packed_bytes))
    for M in Ms:
        sets = len(weights.sets)
        layer = Layer(bl, torch, wl, wname, M, weights)
        cycle, graphs = capture_cycle(torch, layer.decode_step, sets)
        wall, ev_ms = replay_steps(torch, cycle, graphs, steps, warmup)
        step_b = layer.step_bytes()
        # per-step duration from events around replays of 16 steps per graph
        step_us = kernel_avg_us(torch, layer, layer.decode_step, 1, max(steps, 20))
        fwd_b = sum(fwd_bytes(M, *shapes[p]) for p in PROJ)
        fwd_us = kernel_avg_us(torch, layer, layer.forward_fused, 1, max(steps, 20))
        dot4_us = None
        if M <= 4:  # the same forwards with the contraction on v_dot4_i32_i8
            def dot4_fwd(s):
                for _, ps in layer.GROUPS:
                    bl.forward_grouped_dot4([layer.entry(s, p) for p in ps])
            dot4_us = kernel_avg_us(torch, layer, dot4_fwd, 1, max(steps, 20))
        sep_cycle, sep_graphs = capture_cycle(torch, layer.step, sets)
        sep_wall, _ = replay_steps(torch, sep_cycle, sep_graphs, steps, warmup)
        launches = layer.fused_launches()
        r = {"ms_per_step": 1e3 * wall / steps, "event_ms_per_step": ev_ms / steps, "step_bytes": step_b,
             "step_us": step_us, "step_gbs": step_b / (step_us * 1e-6) / 1e9,
             "step_frac_hbm": step_b / (step_us * 1e-6) / 1e9 / PEAK_HBM_GBS, "launches_per_step": launches,
             "bytes_per_launch_avg": step_b / launches, "us_per_launch_avg": step_us / launches,
             "forward_only": {"bytes": fwd_b, "us": fwd_us, "gbs": fwd_b / (fwd_us * 1e-6) / 1e9,
                              "frac_hbm": fwd_b / (fwd_us * 1e-6) / 1e9 / PEAK_HBM_GBS, "launches": 4},
             "forward_only_dot4_us": dot4_us,
             "separate_quant_ms_per_step": 1e3 * sep_wall / steps, "rotation_sets": sets}
        if per_proj:
            per = {}
            for p in PROJ:
                us = kernel_avg_us(torch, layer, lambda s, p=p: layer.forward(s, p), 1, max(steps, 20))
                N, K = shapes[p]
                b = fwd_bytes(M, N, K)
                per[p] = {"N": N, "K": K, "us": us, "gbs": b / (us * 1e-6) / 1e9}
            r["per_projection"] = per
        res[f"M{M}"] = r
        del layer, graphs, cycle, sep_graphs, sep_cycle
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    return res


def bench_decode_b1(bl, torch, wl, wname, Ms, steps, warmup):
    """Binary weights in the one-bit layout b1: the decode step as a serving
    loop runs it (per input, its activation quant and the forwards that read
    it in one call: bitlinear_quant_forward_b1_grouped), the same step with
    separate quant launches (8 launches), and the layer's seven forwards alone
    on quantised inputs (QKV grouped, O, gate+up grouped, down: 4 launches)."""
    res = {}
    shapes = wl.WORKLOADS[wname]["tensors"]
    packed_bytes = sum(bl.packed_bytes_b1(*shapes[p]) for p in PROJ)
    weights = Weights(bl, torch, wl, wname, rotation_sets(packed_bytes), b1=True)
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    for M in Ms:
        sets = len(weights.sets)
        layer = Layer(bl, torch, wl, wname, M, weights)

        def fwd(s):
            for ps in groups:
                bl.forward_b1_grouped([layer.entry(s, p) for p in ps])

        def step_separate(s):
            for i, ps in zip(INPUTS, groups):
                bl.quant_act(layer.x[s][i], xq=layer.q[s][i][0], x_scale=layer.q[s][i][1])
                bl.forward_b1_grouped([layer.entry(s, p) for p in ps])

        def step(s):
            for ps in groups:
                bl.quant_forward_b1_grouped([layer.qentry(s, p) for p in ps])

        step(0)
        step_separate(0)
        torch.cuda.synchronize()
        fwd_b = sum(fwd_bytes_b1(M, *shapes[p]) for p in PROJ)
        fwd_us = kernel_avg_us(torch, layer, fwd, 1, max(steps, 20))
        step_b = fwd_b + sum(quant_bytes(M, layer.kin[i]) for i in INPUTS)
        step_us = kernel_avg_us(torch, layer, step, 1, max(steps, 20))
        sep_us = kernel_avg_us(torch, layer, step_separate, 1, max(steps, 20))
        per = {}
        for p in PROJ:
            us = kernel_avg_us(torch, layer, lambda s, p=p: bl.forward_b1_grouped([layer.entry(s, p)]), 1,
                               max(steps, 20))
            N, K = shapes[p]
            per[p] = {"N": N, "K": K, "us": us, "gbs": fwd_bytes_b1(M, N, K) / (us * 1e-6) / 1e9}
        res[f"M{M}"] = {"forward_only": {"bytes": fwd_b, "us": fwd_us, "gbs": fwd_b / (fwd_us * 1e-6) / 1e9,
                                         "frac_hbm": fwd_b / (fwd_us * 1e-6) / 1e9 / PEAK_HBM_GBS, "launches": 4},
                        "step": {"bytes": step_b, "us": step_us, "gbs": step_b / (step_us * 1e-6) / 1e9,
                                 "frac_hbm": step_b / (step_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                 "launches": layer.fused_launches()},
                        "step_separate_quant_us": sep_us,
                        "per_projection": per, "rotation_sets": sets}
        del layer
        torch.cuda.empty_cache()
    del weights
    torch.cuda.empty_cache()
    return res


def load_peaks():
    import ctypes as C
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbench_peaks.so")
    if not os.path.exists(path):
        return None
    L = C.CDLL(path)
    L.peaks_read.argtypes = [C.c_void_p, C.c_int64, C.c_void_p, C.c_int, C.c_void_p]
    L.peaks_mfma_i8.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p]
    return L


def bench_peaks(torch, steps):
    """Measured ceilings on this GPU: HBM read bandwidth (a 2 GiB buffer, 8x
    the last-level cache, streamed once per launch), a device-to-device copy
    (torch, 1 GiB each way), int8 MFMA throughput (32x32x32 from registers),
    and the time per launch of an empty-body graph node."""
    L = load_peaks()
    if L is None:
        return None
    import ctypes as C
    stream = torch.cuda.current_stream()
    sptr = C.c_void_p(stream.cuda_stream)
    out = {}
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    blocks = 256 * 16
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    reps = max(5, steps // 5)
    t = timed(lambda: L.peaks_read(C.c_void_p(buf.data_ptr()), nbytes, C.c_void_p(sink.data_ptr()), blocks, sptr),
              reps)
    out["hbm_read_gbs"] = nbytes / t / 1e9
    a = buf[: nbytes // 2]
    b = buf[nbytes // 2:]
    t = timed(lambda: b.copy_(a), reps)
    out["hbm_copy_gbs"] = nbytes / t / 1e9  # bytes read + written
    del buf, a, b
    torch.cuda.empty_cache()
    iters, mblocks = 4096, 256 * 2
    t = timed(lambda: L.peaks_mfma_i8(iters, mblocks, C.c_void_p(sink.data_ptr()), sptr), 5)
    out["int8_mfma_tops"] = mblocks * 4 * iters * 8 * 65536 / t / 1e12
    out["int8_mfma_config"] = f"{mblocks} workgroups x 4 waves x {iters} x 8 v_mfma_i32_32x32x32_i8"
    # launch cost of a graph node that does nothing (an empty copy stands in)
    z = torch.zeros(1, device="cuda")
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    s2.wait_stream(stream)
    with torch.cuda.stream(s2):
        z.add_(0.0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(64):
            z.add_(0.0)
    t = timed(lambda: g.replay(), 20)
    out["graph_node_us"] = t / 64 * 1e6
    # the stream-read floor of one launch of a given size (the sizes of the
    # decode launches: 3B O, 70B Q, QKV, down, gate+up), timed like them:
    # events around graph replays of many launches, cycling through slices
    # of a buffer larger than twice the last-level cache
    sizes = {"2.56MB": 2_560_000, "8.4MB": 8_388_608, "16.8MB": 16_777_216, "21MB": 20_971_520,
             "58.7MB": 58_720_256, "117MB": 117_440_512}
    span = 1 << 30
    rb = torch.empty(span + (128 << 20), dtype=torch.uint8, device="cuda")
    rb.fill_(1)
    floor = {}
    for name, sz in sizes.items():
        nsl = max(16, -(-2 * MALL_BYTES // sz))
        nsl = min(nsl, (span + (128 << 20)) // sz)
        blk = int(min(2048, max(1, sz // (16 * 256 * 4))))
        gs = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s2):
            L.peaks_read(C.c_void_p(rb.data_ptr()), sz, C.c_void_p(sink.data_ptr()), blk, C.c_void_p(s2.cuda_stream))
        torch.cuda.synchronize()
        with torch.cuda.graph(gs):
            cs = C.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(nsl):
                L.peaks_read(C.c_void_p(rb.data_ptr() + i * sz), sz, C.c_void_p(sink.data_ptr()), blk, cs)
        t = timed(lambda: gs.replay(), 5) / nsl
        floor[name] = {"us": t * 1e6, "gbs": sz / t / 1e9}
        del gs
    out["hbm_read_by_size"] = floor
    del rb
    torch.cuda.empty_cache()
    out["published"] = {"hbm_gbs": PEAK_HBM_GBS, "int8_tops": PEAK_INT8_TOPS}
    return out


def kernel_launches(torch, fn):
    """Kernel launches one call of fn makes: the kernel nodes of a HIP graph
    captured around it (None where the graph cannot be inspected)."""
    import ctypes as C
    try:
        hip = C.CDLL("libamdhip64.so")
        g = torch.cuda.CUDAGraph(keep_graph=True)
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(g, stream=st):
            fn()
        torch.cuda.synchronize()
        raw = C.c_void_p(g.raw_cuda_graph())
        n = C.c_size_t(0)
        if hip.hipGraphGetNodes(raw, None, C.byref(n)) != 0:
            return None
        nodes = (C.c_void_p * n.value)()
        if hip.hipGraphGetNodes(raw, nodes, C.byref(n)) != 0:
            return None
        kinds = C.c_int(0)
        count = 0
        for nd in nodes[: n.value]:
            if hip.hipGraphNodeGetType(C.c_void_p(nd), C.byref(kinds)) != 0:
                return None
            count += kinds.value == 0  # hipGraphNodeTypeKernel
        del g
        return count
    except Exception:
        return None


def bench_linear(bl, torch, wl, steps, warmup):
    """The single BitLinear of K=256 -> N=512 at M=32 tokens (73,860
    algorithmic bytes, 8.4e6 ops: latency-bound).  Absolute microseconds per
    call from events around graph replays of 64 back-to-back calls: the
    activation quant and the forward as one call, and the forward alone on
    quantised tokens."""
    N, K = wl.WORKLOADS["linear_256x512"]["tensors"]["w"]
    M = 32
    W = torch.from_numpy(wl.workload_weight("linear_256x512", "w")).cuda()
    packed, g = bl.pack_weights(W)
    x = torch.from_numpy(wl.workload_activation("linear_256x512", "w", M).view(np.int16)).cuda().view(torch.bfloat16)
    xq, xs = bl.quant_act(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ent = dict(packed=packed, gamma=g, N=N, K=K, x=x, xq=xq, x_scale=xs, y=y)

    def qf(_s):
        for _ in range(64):
            bl.quant_forward_grouped([ent])

    def fw(_s):
        for _ in range(64):
            bl.forward(packed, g, N, K, xq, xs, y=y, workspace=None)

    out = {"M": M, "N": N, "K": K, "bytes": fwd_bytes(M, N, K), "ops": fwd_ops(M, N, K)}
    for label, fn in (("quant_forward_us", qf), ("forward_us", fw)):
        gr = capture(torch, fn, 1)
        n = max(4, steps // 4)
        _, ms = replay_timed(torch, gr, n, 2)
        out[label] = ms * 1e3 / (n * 64)
    out["launches_quant_forward"] = kernel_launches(torch, lambda: bl.quant_forward_grouped([ent]))
    return out


def bench_model16m(bl, torch, wl, steps, warmup):
    """The 42 BitLinear tensors of the 6-layer model (hidden 256, 4/2 heads of
    64, SwiGLU 512) at 8192 tokens (32 sequences x 256): per layer QKV
    (grouped), O, gate+up (grouped), down.  Forward GB/s over the algorithmic
    bytes of the 42 forwards (304.3 MB, bound by the bf16 output), and the
    step with the 24 activation quants."""
    name = "model_16m"
    M = 8192
    shapes = wl.WORKLOADS[name]["tensors"]
    per_set = sum(fwd_bytes(M, *shapes[p]) for p in PROJ) * 6
    sets = rotation_sets(per_set)
    layers = [Layer(bl, torch, wl, name, M, Weights(bl, torch, wl, name, sets, layer=l)) for l in range(6)]

    def fwd(s):
        for ly in layers:
            ly.forward_fused(s)

    def step(s):
        for ly in layers:
            ly.step(s)

    for ly in layers:
        for s in range(sets):
            ly.quant(s)
    fb = 6 * sum(fwd_bytes(M, *shapes[p]) for p in PROJ)
    sb = fb + 6 * sum(quant_bytes(M, layers[0].kin[i]) for i in INPUTS)
    fwd_us = kernel_avg_us(torch, layers[0], fwd, 1, max(steps, 20))
    step_us = kernel_avg_us(torch, layers[0], step, 1, max(steps, 20))
    out = {"M": M, "tensors": 42, "rotation_sets": sets,
           "forward": {"bytes": fb, "us": fwd_us, "gbs": fb / (fwd_us * 1e-6) / 1e9,
                       "frac_hbm": fb / (fwd_us * 1e-6) / 1e9 / PEAK_HBM_GBS, "launches": 24,
                       "ops": 6 * sum(fwd_ops(M, *shapes[p]) for p in PROJ)},
           "with_quant": {"bytes": sb, "us": step_us, "gbs": sb / (step_us * 1e-6) / 1e9, "launches": 48}}
    del layers
    torch.cuda.empty_cache()
    return out


def bench_aux(bl, torch, wl, steps, warmup):
    """Pack of all 42 tensors of the 6-layer model (one grouped call: three
    launches per 16 tensors; and 42 separate calls for reference), and one
    tracker update over their 3,538,944 weights held as one flat buffer."""
    tl = wl.workload_tensors("model_16m")
    Ws = [torch.from_numpy(wl.workload_weight("model_16m", p, l)).cuda() for (l, p, N, K) in tl]
    outs = [(torch.empty(bl.packed_bytes(N, K), dtype=torch.uint8, device="cuda"),
             torch.empty(1, dtype=torch.float32, device="cuda"),
             torch.empty(bl.pack_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")) for (l, p, N, K) in tl]

    def pack_all(_s):
        for W, (pk, g, ws) in zip(Ws, outs):
            bl.pack_weights(W, packed=pk, gamma=g, workspace=ws)

    def pack_grouped(_s):
        bl.pack_weights_grouped(Ws, outs=[(pk, g) for pk, g, _ in outs], workspaces=[ws for _, _, ws in outs])

    n_w = sum(N * K for (l, p, N, K) in tl)
    g_pack = capture(torch, pack_grouped, 1)
    _, ms = replay_timed(torch, g_pack, steps, warmup)
    pack_us = ms * 1e3 / steps
    g_sep = capture(torch, pack_all, 1)
    _, ms = replay_timed(torch, g_sep, steps, warmup)
    sep_us = ms * 1e3 / steps
    pack = {"tensors": len(tl), "weights": n_w, "us_per_pass": pack_us, "launches": 9,
            "gbs_two_pass": n_w * 8.25 / (pack_us * 1e-6) / 1e9,
            "separate_calls_us_per_pass": sep_us, "separate_launches": 3 * len(tl)}

    prev, curr, mask = wl.flip_snapshots("model_16m")
    fc0, lf0, step = wl.flip_counters(prev.size, 2)
    tsets = rotation_sets(prev.size * 12)  # 8 B of snapshots + 4 B of counters per weight resident
    bufs = [(torch.from_numpy(prev).cuda(), torch.from_numpy(curr).cuda(), torch.from_numpy(fc0).cuda(),
             torch.from_numpy(lf0).cuda()) for _ in range(tsets)]

    def flip(_s):
        for i in range(16):  # 16 launches per replay, cycling the rotation sets
            pd, cd, fcd, lfd = bufs[i % tsets]
            bl.flip_update(pd, cd, step, fcd, lfd)

    g_flip = capture(torch, flip, 1)
    n_rep = max(2, steps // 4)
    _, ms = replay_timed(torch, g_flip, n_rep, warmup)
    fl_us = ms * 1e3 / (n_rep * 16)
    tracker = {"weights": int(prev.size), "us": fl_us, "gbs": prev.size * 16 / (fl_us * 1e-6) / 1e9,
               "rotation_sets": tsets, "launches_per_replay": 16}
    # read-out: sign age and flip rate from the counters (4 B read + 8 B written per weight)
    fcd, lfd = bufs[0][2], bufs[0][3]
    age = torch.empty(prev.size, dtype=torch.float32, device="cuda")
    rate = torch.empty(prev.size, dtype=torch.float32, device="cuda")

    def stats(_s):
        for _ in range(16):
            bl.flip_stats(fcd, lfd, step, sign_age=age, flip_rate=rate)

    g_st = capture(torch, stats, 1)
    _, ms = replay_timed(torch, g_st, n_rep, warmup)
    st_us = ms * 1e3 / (n_rep * 16)
    tracker["readout_us"] = st_us
    tracker["readout_gbs"] = prev.size * 12 / (st_us * 1e-6) / 1e9
    del bufs, age, rate
    # one 70B FFN matrix (28672 x 8192 fp32, 940 MB): ternary and binary packing
    N, K = wl.WORKLOADS["layer_70b"]["tensors"]["gate"]
    W = torch.randn(N, K, device="cuda", generator=torch.Generator(device="cuda").manual_seed(0)) * 0.02
    pk = torch.empty(bl.packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    sc2 = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(bl.pack_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    big = {}
    for label, fn, bpw in (("ternary", lambda: bl.pack_weights(W, packed=pk, gamma=sc, workspace=ws), 8.25),
                           ("binary", lambda: bl.pack_binary(W, packed=pk, beta=sc, alpha=sc2, workspace=ws), 12.25)):
        g_pk = capture(torch, lambda _s: fn(), 1)
        _, ms = replay_timed(torch, g_pk, max(2, steps // 10), 2)
        us = ms * 1e3 / max(2, steps // 10)
        big[label] = {"us": us, "bytes_per_weight": bpw, "gbs": N * K * bpw / (us * 1e-6) / 1e9}
    pack["70B_ffn_matrix"] = dict(N=N, K=K, **big)
    del W, pk, ws
    torch.cuda.empty_cache()
    return pack, tracker


def bench_optim(bl, torch, wl, steps, warmup):
    """AdamW step with the tracker fused, on one 70B FFN matrix (28672 x 8192
    fp32 shadow weights, optimiser state and gradient: 3.8 GB), next to the
    same update done the unfused way: snapshot copy of W, AdamW, then the
    two-snapshot tracker.  Algorithmic bytes per weight: fused 28 (W, g, m, v
    read; W, m, v written; counters only where a sign changed), unfused 28 +
    8 (snapshot) + 16 (tracker)."""
    N, K = wl.WORKLOADS["layer_70b"]["tensors"]["gate"]
    n = N * K
    gen = torch.Generator(device="cuda").manual_seed(1)
    W = torch.randn(n, device="cuda", generator=gen) * 0.02
    g = torch.randn(n, device="cuda", generator=gen) * 2.5e-4
    m = g * 0.1
    v = g * g
    fc = torch.zeros(n, dtype=torch.int16, device="cuda")
    lf = torch.zeros(n, dtype=torch.int16, device="cuda")
    snap = torch.empty_like(W)
    t = 500
    lr = wl.lr_schedule(t)

    def fused(_s):
        bl.adamw_step(W, g, m, v, t, lr, 0.9, 0.999, 1e-8, 0.1, fc, lf)

    def unfused(_s):
        snap.copy_(W)
        bl.adamw_step(W, g, m, v, t, lr, 0.9, 0.999, 1e-8, 0.1)
        bl.flip_update(snap, W, t, fc, lf)

    out = {"N": N, "K": K, "weights": n, "step": t, "lr": lr}
    for label, fn, bpw in (("fused", fused, 28), ("unfused", unfused, 52)):
        gr = capture(torch, fn, 1)
        reps = max(2, steps // 10)
        _, ms = replay_timed(torch, gr, reps, 2)
        us = ms * 1e3 / reps
        out[label] = {"us": us, "bytes_per_weight": bpw, "gbs": n * bpw / (us * 1e-6) / 1e9,
                      "frac_hbm": n * bpw / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    out["speedup"] = out["unfused"]["us"] / out["fused"]["us"]
    del W, g, m, v, fc, lf, snap
    torch.cuda.empty_cache()
    return out


PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s


def bench_backward(bl, torch, wl, steps, warmup):
    """STE backward to the input for one layer: the 700M prefill layer (2048
    tokens) and one layer of the 16.4M training model (8192 tokens).  The dx
    of Q, K and V sum into one buffer (they share the input), gate and up
    into another; O and down write their own.  The layer is timed as four
    launches (Q+K+V and gate+up grouped) and, under "separate", as seven
    single calls that accumulate.  Flops = 2 M N K per projection (bf16 MFMA,
    dense-equivalent); bytes = dy + codes + dx written (+ the dx read of an
    accumulating single call)."""
    out = {}
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    for name, wname, M in (("700M_prefill", "layer_700m", 2048), ("16M_training", "model_16m", 8192)):
        shapes = wl.WORKLOADS[wname]["tensors"]
        wts = {}
        for p in PROJ:
            N, K = shapes[p]
            pk, g = bl.pack_weights(torch.from_numpy(wl.workload_weight(wname, p)).cuda())
            wts[p] = (bl.pack_transposed(pk, N, K), g, N, K)
        flops = sum(2 * M * shapes[p][0] * shapes[p][1] for p in PROJ)
        nbytes = 0
        for grp in groups:
            for i, p in enumerate(grp):
                N, K = shapes[p]
                nbytes += M * N * 2 + M * K * 2 * (2 if i else 1) + bl.packed_bytes(K, N)
        sets = min(rotation_sets(nbytes), 16)
        gen = torch.Generator(device="cuda").manual_seed(5)
        bufs = []
        for _ in range(sets):
            dys = {p: torch.randn(M, shapes[p][0], device="cuda", generator=gen).to(torch.bfloat16) for p in PROJ}
            dxs = {grp: torch.empty(M, shapes[grp[0]][1], device="cuda", dtype=torch.bfloat16) for grp in groups}
            bufs.append((dys, dxs))

        def one(p, grp, i, si):
            pt, g, N, K = wts[p]
            dys, dxs = bufs[si]
            bl.backward_input(pt, g, N, K, dys[p], dx=dxs[grp], accumulate=i > 0)

        def layer(si):
            for grp in groups:
                for i, p in enumerate(grp):
                    one(p, grp, i, si)

        def body(_s):
            for k in range(16):
                layer(k % sets)

        gr = capture(torch, body, 1)
        n = max(2, steps // 4)
        _, ms = replay_timed(torch, gr, n, warmup)
        us = ms * 1e3 / (n * 16)
        r = {"M": M, "flops": flops, "rotation_sets": sets,
             "separate": {"us_per_layer": us, "bytes": nbytes, "tflops": flops / us / 1e6,
                          "frac_bf16": flops / us / 1e6 / PEAK_BF16_TFLOPS, "gbs": nbytes / us / 1e3,
                          "frac_hbm": nbytes / us / 1e3 / PEAK_HBM_GBS, "launches": 7}}
        per = {}
        for grp in groups:
            for i, p in enumerate(grp):
                def body_p(_s, p=p, grp=grp, i=i):
                    for k in range(16):
                        one(p, grp, i, k % sets)
                gp = capture(torch, body_p, 1)
                _, ms = replay_timed(torch, gp, n, 2)
                up = ms * 1e3 / (n * 16)
                N, K = shapes[p]
                per[p] = {"N": N, "K": K, "us": up, "tflops": 2 * M * N * K / up / 1e6, "accumulate": i > 0}
        r["per_projection"] = per

        # the layers that read one input summed in one grouped call each
        def one_group(grp, si):
            dys, dxs = bufs[si]
            if len(grp) == 1:
                one(grp[0], grp, 0, si)
                return
            ents = [(wts[p][0], wts[p][1], wts[p][2], dys[p]) for p in grp]
            bl.backward_input_grouped(ents, wts[grp[0]][3], dx=dxs[grp])

        def body_g(_s):
            for k in range(16):
                for grp in groups:
                    one_group(grp, k % sets)

        gg = capture(torch, body_g, 1)
        _, ms = replay_timed(torch, gg, n, warmup)
        ug = ms * 1e3 / (n * 16)
        # one dx write per group, no dx reads
        gbytes = sum(M * shapes[p][0] * 2 + bl.packed_bytes(shapes[p][1], shapes[p][0]) for p in PROJ) + \
            sum(M * shapes[grp[0]][1] * 2 for grp in groups)
        r.update({"us_per_layer": ug, "bytes": gbytes, "tflops": flops / ug / 1e6,
                  "frac_bf16": flops / ug / 1e6 / PEAK_BF16_TFLOPS, "gbs": gbytes / ug / 1e3,
                  "frac_hbm": gbytes / ug / 1e3 / PEAK_HBM_GBS, "launches": len(groups)})
        per_g = {}
        for grp in groups:
            if len(grp) == 1:
                continue
            def body_pg(_s, grp=grp):
                for k in range(16):
                    one_group(grp, k % sets)
            gp = capture(torch, body_pg, 1)
            _, ms = replay_timed(torch, gp, n, 2)
            up = ms * 1e3 / (n * 16)
            fl = sum(2 * M * shapes[p][0] * shapes[p][1] for p in grp)
            per_g["+".join(grp)] = {"us": up, "tflops": fl / up / 1e6,
                                    "us_separate": sum(per[p]["us"] for p in grp)}
        r["per_group"] = per_g
        out[name] = r
        del bufs, wts
        torch.cuda.empty_cache()
    return out


def bench_norm(bl, torch, wl, steps, warmup):
    """RMSNorm fused into the activation quant (the step before a layer's
    first forward) next to the plain quant, on the 700M prefill input
    (2048 x 1536) and a 70B decode input (1 x 8192); bytes = 3 M K + 4 M + 4 K."""
    out = {}
    for name, (M, K, key) in {"700M_prefill": (2048, 1536, (3, 0)), "70B_decode": (1, 8192, (5, 0)),
                              "70B_decode_M64": (64, 8192, (5, 1))}.items():
        x = wl.activation(M, K, key=(1600,) + key, recipe="plain")
        gain = torch.from_numpy(np.float32(1.0) + np.float32(0.1) * wl.rng(1601, K).standard_normal(K, dtype=np.float32)).cuda()
        sets = min(rotation_sets(3 * M * K + 4 * M), 64)  # tiny rows are latency-bound, not cached
        xs = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for _ in range(sets)]
        qs = [(torch.empty((M, K), dtype=torch.int8, device="cuda"), torch.empty(M, dtype=torch.float32, device="cuda"))
              for _ in range(sets)]

        def norm(_s):
            for i in range(16):
                bl.rmsnorm_quant_act(xs[i % sets], gain=gain, xq=qs[i % sets][0], x_scale=qs[i % sets][1])

        def plain(_s):
            for i in range(16):
                bl.quant_act(xs[i % sets], xq=qs[i % sets][0], x_scale=qs[i % sets][1])

        r = {"M": M, "K": K, "rotation_sets": sets}
        for label, fn in (("fused_norm_quant", norm), ("plain_quant", plain)):
            g = capture(torch, fn, 1)
            n = max(2, steps // 4)
            _, ms = replay_timed(torch, g, n, warmup)
            us = ms * 1e3 / (n * 16)
            b = 3 * M * K + 4 * M + (4 * K if label == "fused_norm_quant" else 0)
            r[label] = {"us": us, "gbs": b / (us * 1e-6) / 1e9, "frac_hbm": b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
        out[name] = r
        del xs, qs
        torch.cuda.empty_cache()
    return out


def cpu_baseline(wl, target_s=12.0):
    """The oracle on the GPU machine's host cores, each step timed on its own:
    pack (gamma + ternarise + layout) of the 700M layer's Q weight; the
    activation quant and the contraction + rescale of all 7 projections on
    the first T of the 2048 prefill tokens (T doubled until a run takes a few
    seconds); the sign-flip tracker over the 6-layer model's 3,538,944
    weights.  The headline value is quant + contraction + rescale in TOPS, on
    all host threads, then on one thread with a smaller T."""
    import oracle
    shapes = wl.WORKLOADS["layer_700m"]["tensors"]
    rep = {"qkv": "q", "o": "o", "gateup": "gate", "down": "down"}
    inp_of = {"q": "qkv", "k": "qkv", "v": "qkv", "o": "o", "gate": "gateup", "up": "gateup", "down": "down"}
    codes, gam = {}, {}
    t_pack, n_pack = 0.0, 0
    for p in PROJ:
        W = wl.workload_weight("layer_700m", p)
        t0 = time.perf_counter()
        pk, g, c = oracle.pack(W)
        if p == "q":
            t_pack, n_pack = time.perf_counter() - t0, W.size
        codes[p], gam[p] = c, g
    xs = {i: wl.workload_activation("layer_700m", rep[i], 2048) for i in INPUTS}

    def run(target):
        T = 4
        while True:
            t0 = time.perf_counter()
            qs = {i: oracle.quant_act(xs[i][:T]) for i in INPUTS}
            t1 = time.perf_counter()
            for p in PROJ:
                q, s_ = qs[inp_of[p]]
                oracle.epilogue(oracle.contract(q, codes[p]), gam[p], s_)
            t2 = time.perf_counter()
            if (t2 - t0) * 2 > target or T >= 2048:
                return T, t1 - t0, t2 - t1
            T *= 2

    T, tq, tc = run(target_s)
    ops = sum(fwd_ops(T, *shapes[p]) for p in PROJ)
    qb = sum(quant_bytes(T, shapes[rep[i]][1]) for i in INPUTS)
    prev, curr, _ = wl.flip_snapshots("model_16m")
    fc, lf, step = wl.flip_counters(prev.size, 2)
    t0 = time.perf_counter()
    oracle.flip_update(prev, curr, step, fc, lf)
    t_flip = time.perf_counter() - t0
    all_threads = oracle.threads()
    oracle.set_threads(1)  # the same job on one host thread, a smaller sample
    try:
        T1, tq1, tc1 = run(target_s / 3)
    finally:
        oracle.set_threads(all_threads)
    ops1 = sum(fwd_ops(T1, *shapes[p]) for p in PROJ)
    import platform
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": ops / (tq + tc) / 1e12, "unit": "TOPS", "cores": all_threads, "kind": "oracle",
            "sample": f"700M layer prefill, first {T} of 2048 tokens, all 7 projections "
                      f"(quant + add/subtract/skip contraction + rescale), {tq + tc:.2f} s",
            "steps": {
                "pack": {"weights": n_pack, "s": t_pack, "weights_per_s": n_pack / t_pack, "threads": 1,
                         "sample": "700M layer Q weight (1536 x 1536): gamma, ternarise, layout v1"},
                "quant": {"tokens": T, "s": tq, "gbs": qb / tq / 1e9, "threads": 1,
                          "sample": f"the 4 layer inputs, first {T} tokens"},
                "contract_epilogue": {"tokens": T, "s": tc, "tops": ops / tc / 1e12, "threads": all_threads},
                "tracker": {"weights": int(prev.size), "s": t_flip, "gbs": prev.size * 16 / t_flip / 1e9,
                            "threads": 1, "sample": "6-layer model, 42 tensors, pre-seeded counters, step 1000"}},
            "one_thread": {"value": ops1 / (tq1 + tc1) / 1e12, "unit": "TOPS", "cores": 1,
                           "sample": f"the same job on the first {T1} tokens, {tq1 + tc1:.2f} s"},
            "cpu": cpu, "machine": platform.machine()}


DECODE_LAYERS = {"70B": "layer_70b", "3B": "layer_3b"}
COPY_BYTES = 512 << 20
TRAFFIC_FILE = os.path.join("profiles", "traffic_prefill700m_decode70b.txt")
# the sources of the two kernels whose traffic the counters measured
KERNEL_SOURCES = ("csrc/device.h", "csrc/internal.h", "csrc/gemm_pipe.hip", "csrc/gemv.hip")


def parse_decode(spec):
    out = []
    for part in filter(None, spec.split(";")):
        name, ms = part.split(":")
        if name not in DECODE_LAYERS:
            raise SystemExit(f"unknown decode layer {name!r} (known: {sorted(DECODE_LAYERS)})")
        out.append((name, tuple(int(m) for m in ms.split(","))))
    return out


def kernel_source_hash(root):
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, "bitlinear_absmean_ternarise_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(root, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size).  Empty
    when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(root, TRAFFIC_FILE)
    if not os.path.exists(path):
        return {}
    rec, src = {}, None
    with open(path) as f:
        for ln in f:
            parts = ln.split()
            if len(parts) == 2 and parts[0] == "kernel_source_sha256:":
                src = parts[1]
            elif len(parts) == 3 and parts[0] == "traffic_bytes_per_launch:":
                rec[parts[1]] = float(parts[2])
    if src != kernel_source_hash(root) or kernel not in rec:
        return {}
    return {"bytes_per_launch": rec[kernel], "source": f"{TRAFFIC_FILE} (kernel sources {src})"}


def eager_kernels(bl, torch, wl, reps, which="all"):
    """Launch each measured kernel `reps` times per rotation set without graphs
    and without timing, so a counter-collecting profiler sees every dispatch:
    a plain copy of COPY_BYTES (the calibration), the grouped prefill forwards
    of the 700M layer at M=2048 (gemm_pipe), and the 70B M=1 decode step
    (quant + forward in one launch per input: gemv_quant16)."""
    n = COPY_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    del a, b
    print(f"# copy: {reps} x {COPY_BYTES} bytes read + written (torch.neg)", file=sys.stderr, flush=True)
    if which in ("all", "prefill"):
        probe = wl.WORKLOADS["layer_700m"]["tensors"]
        sets = rotation_sets(sum(fwd_bytes(2048, *probe[p]) for p in PROJ))
        layer = Layer(bl, torch, wl, "layer_700m", 2048, Weights(bl, torch, wl, "layer_700m", sets))
        for s in range(sets):
            layer.quant(s)
        for _ in range(reps):
            for s in range(sets):
                layer.forward_fused(s)
        torch.cuda.synchronize()
        print(f"# prefill: {reps} x {sets} sets x 4 grouped launches", file=sys.stderr, flush=True)
        del layer
        torch.cuda.empty_cache()
    if which in ("all", "decode"):
        shapes = wl.WORKLOADS["layer_70b"]["tensors"]
        weights = Weights(bl, torch, wl, "layer_70b", rotation_sets(sum(bl.packed_bytes(*shapes[p]) for p in PROJ)))
        layer = Layer(bl, torch, wl, "layer_70b", 1, weights)
        for _ in range(reps):
            for s in range(len(weights.sets)):
                layer.decode_step(s)
        torch.cuda.synchronize()
        print(f"# decode: {reps} x {len(weights.sets)} sets x {layer.fused_launches()} launches (quant + forward)",
              file=sys.stderr, flush=True)
    if which == "batch":
        # the 70B forwards for a decode batch of 64 tokens (the GEMM with K cut
        # into runs and the reduce), 4 launches + reduces per set
        shapes = wl.WORKLOADS["layer_70b"]["tensors"]
        weights = Weights(bl, torch, wl, "layer_70b", rotation_sets(sum(bl.packed_bytes(*shapes[p]) for p in PROJ)))
        layer = Layer(bl, torch, wl, "layer_70b", 64, weights)
        for s in range(len(weights.sets)):
            layer.quant(s)
        for _ in range(reps):
            for s in range(len(weights.sets)):
                layer.forward_fused(s)
        torch.cuda.synchronize()
        print(f"# batch forwards (M=64): {reps} x {len(weights.sets)} sets", file=sys.stderr, flush=True)
    if which == "forwards":
        # the 70B M=1 forwards alone on quantised inputs: two-bit (gemv_mfma16)
        # and binary one-bit (gemv_b1) weights, 4 launches per set each
        shapes = wl.WORKLOADS["layer_70b"]["tensors"]
        for b1 in (False, True):
            size = bl.packed_bytes_b1 if b1 else bl.packed_bytes
            weights = Weights(bl, torch, wl, "layer_70b", rotation_sets(sum(size(*shapes[p]) for p in PROJ)), b1=b1)
            layer = Layer(bl, torch, wl, "layer_70b", 1, weights)
            for s in range(len(weights.sets)):
                layer.quant(s)
            for _ in range(reps):
                for s in range(len(weights.sets)):
                    if b1:
                        for ps in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",)):
                            bl.forward_b1_grouped([layer.entry(s, p) for p in ps])
                    else:
                        layer.forward_fused(s)
            torch.cuda.synchronize()
            print(f"# forwards ({'one-bit binary' if b1 else 'two-bit'}): {reps} x {len(weights.sets)} sets x 4 "
                  "launches", file=sys.stderr, flush=True)
            del layer, weights
            torch.cuda.empty_cache()


def _round(o, nd=4):
    """Floats rounded for the summary line (big ints kept)."""
    if isinstance(o, float):
        return float(f"{o:.{nd}g}") if abs(o) < 1e6 else round(o, 1)
    if isinstance(o, dict):
        return {k: _round(v, nd) for k, v in o.items()}
    if isinstance(o, (list, tuple)):
        return [_round(v, nd) for v in o]
    return o


def decode_summary(dec):
    """Compact per-configuration decode record for the summary line."""
    out = {}
    for name, res in dec.items():
        for key, r in res.items():
            out[f"{name} {key.replace('M', 'M=')}"] = _round({
                "step_us": r["step_us"], "step_gbs": r["step_gbs"], "step_frac_hbm": r["step_frac_hbm"],
                "launches": r["launches_per_step"], "step_bytes": r["step_bytes"],
                "forward_only_us": r["forward_only"]["us"], "forward_only_gbs": r["forward_only"]["gbs"],
                "forward_only_dot4_us": r.get("forward_only_dot4_us"),
                "separate_quant_step_us": 1e3 * r["separate_quant_ms_per_step"]})
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the BitLinear path is measured on a "
                                   "single MI355X (multi-GPU sharding is a design note, not built)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    import torch
    import bitlinear_absmean_ternarise_amd as bl
    import workloads as wl
    assert torch.cuda.is_available(), "no GPU visible"
    torch.manual_seed(0)
    dev = torch.cuda.get_device_properties(0)
    print(f"# device {dev.name} {getattr(dev, 'gcnArchName', '')}", file=sys.stderr, flush=True)

    if args.eager_kernels:
        eager_kernels(bl, torch, wl, args.eager_kernels, args.eager_only)
        return

    full = args.only is None and not args.quick
    peaks = None
    if full or args.only == "peaks":
        print("# measured peaks (HBM read, copy, int8 MFMA, graph node)", file=sys.stderr, flush=True)
        peaks = bench_peaks(torch, args.steps)
    pre = None
    if args.only in (None, "prefill"):
        print("# prefill (700M layer, M=2048)", file=sys.stderr, flush=True)
        pre = bench_prefill(bl, torch, wl, args.steps, args.warmup, per_proj=not args.no_per_proj)
    dec = {}
    if not args.quick and args.only in (None, "decode"):
        for name, Ms in parse_decode(args.decode):
            print(f"# decode {name} layer, M={Ms}", file=sys.stderr, flush=True)
            dec[name] = bench_decode(bl, torch, wl, DECODE_LAYERS[name], Ms, args.steps, args.warmup,
                                     per_proj=not args.no_per_proj)
    b1 = {}
    if full or args.only == "b1":
        for name, Ms in parse_decode(args.b1):
            print(f"# decode {name} layer, binary weights in the one-bit layout, M={Ms}", file=sys.stderr, flush=True)
            b1[name] = bench_decode_b1(bl, torch, wl, DECODE_LAYERS[name], Ms, args.steps, args.warmup)
    lin = m16 = None
    if full or args.only == "small":
        print("# single BitLinear 256 -> 512, M=32", file=sys.stderr, flush=True)
        lin = bench_linear(bl, torch, wl, args.steps, args.warmup)
        print("# 6-layer model, 42 tensors, M=8192", file=sys.stderr, flush=True)
        m16 = bench_model16m(bl, torch, wl, args.steps, args.warmup)
    pack = tracker = norm = optim = bwd = None
    if full or args.only == "aux":
        print("# pack + tracker (6-layer model)", file=sys.stderr, flush=True)
        pack, tracker = bench_aux(bl, torch, wl, args.steps, args.warmup)
        print("# RMSNorm fused into the quant", file=sys.stderr, flush=True)
        norm = bench_norm(bl, torch, wl, args.steps, args.warmup)
        print("# STE backward to the input", file=sys.stderr, flush=True)
        bwd = bench_backward(bl, torch, wl, args.steps, args.warmup)
        print("# AdamW step + fused tracker (70B FFN matrix)", file=sys.stderr, flush=True)
        optim = bench_optim(bl, torch, wl, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu and not args.quick and pre is not None:
        print("# cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl)

    line = {"metric": METRIC}
    detail = {}
    if pre is not None:
        tr_pre = traffic_record(root, "gemm_pipe")
        line.update({
            "value": round(pre["tops"], 3), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(pre["ms_per_step"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
            "config": {"workload": "700M LLaMA-shape layer prefill: hidden 1536, FFN 4096, M=2048 tokens; "
                                   "per step 4 activation quants + 7 BitLinear forwards (Q,K,V,O,gate,up,down) "
                                   "as quant+QKV (grouped), quant+O, quant+gate+up (grouped), quant+down",
                       "M": 2048, "hidden": 1536, "ffn": 4096, "parallelism": "none (1 GPU)"},
            "roofline": {"bound": "mfma", "achieved": round(pre["gemm_tops"], 3), "peak": PEAK_INT8_TOPS,
                         "unit": "TOPS", "frac": round(pre["gemm_tops"] / PEAK_INT8_TOPS, 5),
                         "traffic": tr_pre.get("bytes_per_launch"),
                         "kernel": "gemm_pipe (int8 MFMA 32x32x32), 4 launches per step: QKV grouped, O, "
                                   "gate+up grouped, down",
                         "traffic_source": tr_pre.get("source"),
                         "ops_per_launch_avg": pre["gemm_ops_per_launch_avg"],
                         "us_per_launch_avg": round(pre["gemm_us_per_launch_avg"], 3)},
        })
        if peaks:
            line["roofline"]["frac_measured_peak"] = round(pre["gemm_tops"] / peaks["int8_mfma_tops"], 5)
    # the decode half of the metric, as short top-level fields
    for name, res in dec.items():
        for key, r in res.items():
            tag = f"decode_{name.lower()}_{key.lower()}"
            line[f"{tag}_gbs"] = round(r["step_gbs"], 1)
            line[f"{tag}_frac_hbm"] = round(r["step_frac_hbm"], 4)
    if lin:
        line["linear_256x512_m32_us"] = round(lin["quant_forward_us"], 3)
    if m16:
        line["model16m_forward_gbs"] = round(m16["forward"]["gbs"], 1)
    if peaks:
        line["peaks"] = _round({k: v for k, v in peaks.items() if k != "published"})
    if dec:
        name = "70B" if "70B" in dec else next(iter(dec))
        key = "M1" if "M1" in dec[name] else next(iter(dec[name]))
        d1 = dec[name][key]
        tr = traffic_record(root, "gemv_quant16")
        line["decode"] = {
            "value": round(d1["step_gbs"], 1), "unit": "GB/s",
            "workload": f"{name} LLaMA-shape layer decode, {key.replace('M', 'M=')}: per input its activation quant "
                        "and the forwards that read it in one call (QKV grouped, O, gate+up grouped, down); "
                        f"{d1['step_bytes'] / 1e6:.1f} MB of algorithmic bytes per step",
            "frac_hbm": round(d1["step_frac_hbm"], 4), "ms_per_step": round(d1["ms_per_step"], 5),
            "roofline": {"bound": "hbm", "achieved": round(d1["step_gbs"], 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(d1["step_frac_hbm"], 4),
                         "traffic": tr.get("bytes_per_launch") if (name, key) == ("70B", "M1") else None,
                         "kernel": f"gemv_quant16 (activation quant + GEMV), {d1['launches_per_step']} launches per step",
                         "bytes_per_launch_avg": d1["bytes_per_launch_avg"],
                         "us_per_launch_avg": round(d1["us_per_launch_avg"], 3),
                         "traffic_source": tr.get("source")},
            "results": decode_summary(dec)}
        if peaks:
            line["decode"]["roofline"]["frac_measured_peak"] = round(d1["step_gbs"] / peaks["hbm_read_gbs"], 4)
        detail["decode"] = dec
    if b1:
        out = {}
        for name, res in b1.items():
            for key, r in res.items():
                f = r["forward_only"]
                e = {"step_us": r["step"]["us"], "step_gbs": r["step"]["gbs"], "step_frac_hbm": r["step"]["frac_hbm"],
                     "step_separate_quant_us": r["step_separate_quant_us"], "forward_us": f["us"],
                     "forward_gbs": f["gbs"], "forward_frac_hbm": f["frac_hbm"]}
                two = dec.get(name, {}).get(key)
                if two:
                    e["two_bit_step_us"] = two["step_us"]
                    e["two_bit_forward_us"] = two["forward_only"]["us"]
                out[f"{name} {key.replace('M', 'M=')}"] = e
        line["decode_b1"] = _round(out)
        detail["decode_b1"] = b1
    if pre is not None:
        line["prefill"] = _round({k: v for k, v in pre.items() if k != "per_projection"})
        detail["prefill"] = pre
    if lin:
        line["linear_256x512"] = _round(lin)
    if m16:
        line["model_16m"] = _round(m16)
    if pack:
        line["pack"] = _round({k: v for k, v in pack.items() if k != "70B_ffn_matrix"})
        line["tracker"] = _round(tracker)
        detail["pack"] = pack
    if norm:
        detail["rmsnorm_quant"] = norm
    if optim:
        line["adamw_tracker"] = _round({k: optim[k] for k in ("fused", "unfused", "speedup")})
        detail["adamw_tracker"] = optim
    if bwd:
        line["backward_input"] = _round({k: {kk: v[kk] for kk in ("us_per_layer", "tflops", "frac_bf16")}
                                         for k, v in bwd.items()})
        detail["backward_input"] = bwd
    if cpu:
        line["cpu_baseline"] = _round(cpu)
    print("# detail " + json.dumps(_round(detail, 6)), file=sys.stderr, flush=True)
    if args.detail_out:
        with open(args.detail_out, "w") as f:
            json.dump({"line": line, "detail": detail}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
