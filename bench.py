#!/usr/bin/env python3
"""Benchmark of the sparse ternary BitLinear forward on one MI355X.

Default workload (decode, 2:4): FFN up 6912x2560 and down 2560x6912 BitNet-2B-like projections,
64 distinct up/down pairs (566 MB of packed weights, more than twice the 256 MB last-level cache,
so every step streams them from HBM), bf16 activations ~ N(0,1).  One step is the decode hot path
for the whole layer stream at batch 1, 4 and 16 tokens: per T, per-token int8 quantization of
the stacked activations of all layers (one grouped act_quant launch for the two K) and one
grouped sparse ternary GEMV launch with fused rescale over all 128 projections (the layers' activations are independent
inputs).  Weights are packed once before timing (inference stores packed weights).  The timed
steps are launched on the stream; the same step captured as a HIP graph is checked bitwise against
the eager run and its replays are timed beside it (graph_ms_per_step).

metric: decode weight GB/s = packed weight bytes streamed per step / step time.

Also in the same JSON line:
  roofline      for the grouped GEMV kernel: algorithmic bytes per launch / mean launch duration,
                the durations taken with HIP events on the launch stream around back-to-back
                launches of each T's group right after the timed region (single launches with
                events around each are reported beside them); HBM traffic per launch from the
                committed rocprofv3 counter summary when it was taken on the current kernel
                source (else null)
  prefill       4096 x 4096 -> 11008 2:4 GEMM (Student-t activations): dense-equivalent int8 TOPS
  six_eight, fourteen_sixteen
                (2N-2):2N through overlapping 2:4 windows vs the dense path, 2048 x 4096 -> 4096
  train_step    the 3B-alike layer set at 8192 tokens: pack, act_quant and forward
  cpu_baseline  the CPU oracle on a bounded sample of the same decode workload
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
SMFMAC_I8_PEAK_TOPS = 10100.0  # MI355X int8 with 2:4 structured sparsity, dense-equivalent
MFMA_I8_PEAK_TOPS = 5000.0     # MI355X dense int8 MFMA
UP = (6912, 2560)
DOWN = (2560, 6912)
N_PAIRS = 64
DECODE_T = (1, 4, 16)
COPY_BYTES = 512 << 20         # plain device copy used to scale HBM byte counters
LAYER_STREAM_LAUNCHES = 100    # back-to-back grouped launches per T in the layer-stream reading
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemv_group_decode_pmc.md")
GROUP_SRC = [os.path.join(ROOT, "sparsity_amd", "csrc", f)
             for f in ("gemv_group.hip", "device_common.hpp", "launch.hpp")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the 6:8, 14:16 and training-step legs")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="(internal) print the CPU oracle baseline as JSON and exit; no GPU use")
    ap.add_argument("--profile-pass",
                    choices=("decode", "prefill", "train", "bwd", "bwdgroup", "fwdgroup",
                             "sparse6", "windows", "chain"),
                    default=None,
                    help="for hardware-counter runs, no graph and no JSON line.  decode: two eager "
                         "decode steps, then a plain copy of COPY_BYTES (the counters' scale "
                         "reference); prefill: the prefill GEMM launched five times; train: the "
                         "training-step leg with two timed steps; bwd: the gate projection's "
                         "backward three times; bwdgroup: the layer set's grouped backward three "
                         "times, then the plain copies; fwdgroup: the layer set's grouped forward "
                         "three times, its seven separate forwards three times, then the plain "
                         "copies; sparse6: the decode workload's SPARSE6 and 2:4 groups twice "
                         "at every T, then the plain copies; windows: the 6:8 leg (window and "
                         "dense GEMMs, 2048 x 4096 -> 4096) with two timed launches each, then "
                         "the plain copies; chain: the 128 decode layers as one dependent chain, "
                         "two launches at every T")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------------
# decode workload
# ---------------------------------------------------------------------------------------------

class Decode:
    """64 packed up/down pairs, per-T stacked activations, and one projection group per T."""

    def __init__(self, S, torch):
        g = torch.Generator(device="cuda")
        g.manual_seed(1000)
        self.mats = []
        for i in range(N_PAIRS):
            for (n, K) in (UP, DOWN):
                W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02)
                codes, meta, gamma = S.pack(W.contiguous(), 2, 4)
                del W
                self.mats.append((n, K, codes, meta, gamma))
        self.packed_bytes = sum(c.numel() + m.numel() for (_, _, c, m, _) in self.mats)
        # activations: for each T, one bf16 [64*T, K] block per K (layer pair i owns rows iT..iT+T)
        self.x, self.q, self.groups, self.ys = {}, {}, {}, {}
        for T in DECODE_T:
            for K in (UP[1], DOWN[1]):
                self.x[(T, K)] = torch.randn((N_PAIRS * T, K), generator=g, device="cuda",
                                             dtype=torch.float32).to(torch.bfloat16).contiguous()
                self.q[(T, K)] = (torch.empty((N_PAIRS * T, K), dtype=torch.int8, device="cuda"),
                                  torch.empty(N_PAIRS * T, dtype=torch.float32, device="cuda"))
            projs = []
            for i, (n, K, codes, meta, gamma) in enumerate(self.mats):
                xq, sc = self.q[(T, K)]
                j = i // 2
                y = torch.empty((T, n), dtype=torch.float32, device="cuda")
                projs.append(dict(xq=xq[j * T:(j + 1) * T], scale=sc[j * T:(j + 1) * T], K=K,
                                  codes=codes, meta=meta, gamma=gamma, n=n, y=y))
            self.ys[T] = [p["y"] for p in projs]
            self.groups[T] = S.FwdGroup(projs)
        # fused variant: the same projections read the bf16 rows and quantize them in-kernel
        self.last_ms_per_step = None        # the timed 2:4 step (stream launches)
        self.last_graph_ms_per_step = None  # the same step as a graph replay: the comparator legs
                                            # are graph-timed and are compared with this one
        self.fused, self.ys_fused = {}, {}
        for T in DECODE_T:
            projs = []
            for i, (n, K, codes, meta, gamma) in enumerate(self.mats):
                j = i // 2
                projs.append(dict(x=self.x[(T, K)][j * T:(j + 1) * T], K=K, codes=codes, meta=meta,
                                  gamma=gamma, n=n,
                                  y=torch.empty((T, n), dtype=torch.float32, device="cuda")))
            self.ys_fused[T] = [p["y"] for p in projs]
            self.fused[T] = S.FusedGroup(projs)
        torch.cuda.synchronize()

    def algorithmic_bytes(self, T):
        """Bytes one group launch must move: packed weights, int8 activations, token scales,
        fp32 outputs and gamma of every projection."""
        return sum(c.numel() + m.numel() + T * K + 4 * T + 4 * T * n + 4
                   for (n, K, c, m, _) in self.mats)

    def algorithmic_bytes_fused(self, T):
        """Bytes one fused launch must move: packed weights, bf16 activations, fp32 outputs, gamma."""
        return sum(c.numel() + m.numel() + 2 * T * K + 4 * T * n + 4
                   for (n, K, c, m, _) in self.mats)

    def step_fused(self, S, events=None):
        """One decode step with quantization fused into the grouped GEMV: one launch per T."""
        for T in DECODE_T:
            if events is not None:
                events[T][0].record()
            self.fused[T]()
            if events is not None:
                events[T][1].record()

    def quantize(self, S, T):
        """The stacked activations of both K at T tokens, one grouped act_quant launch."""
        S.act_quant_group([self.x[(T, K)] for K in (UP[1], DOWN[1])],
                          outs=[self.q[(T, K)] for K in (UP[1], DOWN[1])])

    def step(self, S, events=None):
        """One decode step over the layer stream at every T: quantize the stacked activations
        (one grouped act_quant launch), then one grouped GEMV launch over all 128 projections."""
        for T in DECODE_T:
            self.quantize(S, T)
            if events is not None:
                events[T][0].record()
            self.groups[T]()
            if events is not None:
                events[T][1].record()


def decode_fused_leg(S, torch, D, ref, steps, warmup):
    """The decode step with act_quant fused into the grouped GEMV (bitlinear_fwd_group_fused):
    graph-captured, checked bitwise against the plain step's outputs, timed like the main metric."""
    D.step_fused(S)
    torch.cuda.synchronize()
    for T in DECODE_T:
        for y, r in zip(D.ys_fused[T], ref[T]):
            if not torch.equal(y, r):
                raise RuntimeError("fused decode differs from act_quant + grouped GEMV")
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        D.step_fused(S)
    for _ in range(2):
        for T in DECODE_T:
            for y in D.ys_fused[T]:
                y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for T in DECODE_T:
            for y, r in zip(D.ys_fused[T], ref[T]):
                if not torch.equal(y, r):
                    raise RuntimeError("fused graph replay differs from the plain eager run")
    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    # timed as the plain step is: stream launches, the graph replay beside them
    graph_ms = timed(graph.replay)
    ms = timed(lambda: D.step_fused(S))
    for T in DECODE_T:
        for y, r in zip(D.ys_fused[T], ref[T]):
            if not torch.equal(y, r):
                raise RuntimeError("fused timed steps differ from the plain eager run")
    value = D.packed_bytes * len(DECODE_T) / (ms * 1e-3) / 1e9
    per_T = {T: [] for T in DECODE_T}
    for _ in range(max(1, min(steps, 10))):
        events = {T: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for T in DECODE_T}
        D.step_fused(S, events)
        torch.cuda.synchronize()
        for T in DECODE_T:
            per_T[T].append(events[T][0].elapsed_time(events[T][1]) * 1e-3)
    mean_t = {T: float(np.mean(per_T[T])) for T in DECODE_T}
    algo = {T: D.algorithmic_bytes_fused(T) for T in DECODE_T}
    achieved = sum(algo.values()) / sum(mean_t.values()) / 1e9
    return {"workload": "the decode stream with per-token quantization fused into the grouped "
                        "GEMV: one launch per T, bf16 activations in",
            "metric": "decode weight GB/s", "value": round(value, 1), "unit": "GB/s",
            "ms_per_step": round(ms, 4), "graph_ms_per_step": round(graph_ms, 4),
            "outputs_identical_to_unfused": True,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "kernel": "gemv_group_kernel<SPARSE, fused>",
                         "per_T": {str(T): {"launch_us": round(mean_t[T] * 1e6, 2),
                                            "algorithmic_bytes": algo[T],
                                            "GBps": round(algo[T] / mean_t[T] / 1e9, 1)}
                                   for T in DECODE_T}}}


def _graph_ms(torch, fn, steps, warmup):
    """Capture fn once as a HIP graph; mean ms per replay over `steps` replays."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        fn()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def decode_single_leg(S, torch, D, steps, warmup):
    """The decode stream with one bitlinear_fwd launch per projection (no grouping): the same 128
    projections and pre-quantized activations as the grouped GEMV, 128 launches per T, captured
    as one HIP graph per T.  Its roofline uses the grouped GEMV's algorithmic bytes."""
    out = {}
    for T in DECODE_T:
        projs = []
        for i, (n, K, codes, meta, gamma) in enumerate(D.mats):
            xq, sc = D.q[(T, K)]
            j = i // 2
            projs.append((xq[j * T:(j + 1) * T], sc[j * T:(j + 1) * T], K, codes, meta, gamma, n,
                          torch.empty((T, n), dtype=torch.float32, device="cuda")))

        def run():
            for (xq, sc, K, c, m, ga, n, y) in projs:
                S.fwd(xq, sc, K, c, m, ga, n, out=(y, None))
        ms = _graph_ms(torch, run, steps, warmup)
        algo = D.algorithmic_bytes(T)
        out[str(T)] = {"ms": round(ms, 4), "per_launch_us": round(ms * 1e3 / len(projs), 2),
                       "weight_GBps": round(D.packed_bytes / (ms * 1e-3) / 1e9, 1),
                       "frac": round(algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    return {"workload": "the decode stream with one bitlinear_fwd launch per projection: 128 "
                        "launches per T (graph-captured), pre-quantized independent activations",
            "kernel": "gemv_kernel", "per_T": out}


def decode_chain_leg(S, torch, D, steps, warmup):
    """The decode stream as one dependent chain: up_0, down_0, up_1, ... (128 layers), each
    layer's input the previous layer's fp32 output, starting from a bf16 token row block.
    (a) bitlinear_fwd_chain: one persistent launch quantizing and multiplying every layer;
    (b) the same chain as act_quant_i8 + bitlinear_fwd per layer (256 launches, graph-captured).
    Outputs of (a) and (b) are checked bitwise equal first."""
    out = {}
    layers = [dict(codes=c, meta=m, gamma=ga, n=n, K=K) for (n, K, c, m, ga) in D.mats]
    for T in DECODE_T:
        x0 = D.x[(T, UP[1])][:T]
        ch = S.Chain(layers, T)
        ch(x0)
        if ch.error():
            raise RuntimeError("chain launch reported a barrier timeout")
        ys = [torch.empty((T, ly["n"]), dtype=torch.float32, device="cuda") for ly in layers]
        qs = [(torch.empty((T, ly["K"]), dtype=torch.int8, device="cuda"),
               torch.empty(max(T, 4), dtype=torch.float32, device="cuda")[:T]) for ly in layers]

        def calls():
            inp = x0
            for ly, y, (xq, sc) in zip(layers, ys, qs):
                S.act_quant(inp, out=(xq, sc))
                S.fwd(xq, sc, ly["K"], ly["codes"], ly["meta"], ly["gamma"], ly["n"], out=(y, None))
                inp = y
        calls()
        torch.cuda.synchronize()
        for a, b in zip(ys, ch.ys):
            if not torch.equal(a, b):
                raise RuntimeError("chain output differs from act_quant_i8 + bitlinear_fwd")
        ms_calls = _graph_ms(torch, calls, steps, warmup)
        for _ in range(3):
            ch(x0)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for a, b in ev:
            a.record()
            ch(x0)
            b.record()
        torch.cuda.synchronize()
        if ch.error():
            raise RuntimeError("chain launch reported a barrier timeout")
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        out[str(T)] = {"chain_ms": round(ms, 4), "per_layer_us": round(ms * 1e3 / len(layers), 2),
                       "weight_GBps": round(D.packed_bytes / (ms * 1e-3) / 1e9, 1),
                       "per_layer_calls_ms": round(ms_calls, 4),
                       "speedup_vs_calls": round(ms_calls / ms, 3)}
    return {"workload": "the decode stream as one dependent chain of 128 layers (up_0, down_0, "
                        "up_1, ...; each input the previous fp32 output): one bitlinear_fwd_chain "
                        "launch against act_quant_i8 + bitlinear_fwd per layer (graph-captured)",
            "outputs_identical_to_calls": True, "per_T": out}


def decode_mall_leg(S, torch, D, pairs=24, launches=100):
    """The decode layer stream shrunk to fit the 256 MB last-level cache: the first `pairs` up/down
    pairs (212 MB of packed weights for 24) in one grouped launch at T = 1, repeated back to back.
    The kernel's weight loads are non-temporal (each byte is read once per launch), so the cache
    is not kept warm between launches: this reading shows what a cache-sized stream gets with
    them (456 work items for 512 block slots)."""
    xq, sc = D.q[(1, UP[1])]
    xd, sd = D.q[(1, DOWN[1])]
    projs = []
    for i, (n, K, codes, meta, gamma) in enumerate(D.mats[:2 * pairs]):
        j = i // 2
        q, s = (xq, sc) if K == UP[1] else (xd, sd)
        projs.append(dict(xq=q[j:j + 1], scale=s[j:j + 1], K=K, codes=codes, meta=meta,
                          gamma=gamma, n=n, y=torch.empty((1, n), dtype=torch.float32, device="cuda")))
    grp = S.FwdGroup(projs)
    for _ in range(5):
        grp()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        grp()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / launches
    wbytes = sum(c.numel() + m.numel() for (_, _, c, m, _) in D.mats[:2 * pairs])
    return {"workload": f"first {pairs} up/down pairs of the decode stream, T = 1, one grouped launch "
                        f"repeated {launches} times back to back (weights sized to fit the "
                        "last-level cache)",
            "label": "MALL-sized (non-temporal weight loads: not kept resident)",
            "packed_weight_bytes": wbytes,
            "launch_us": round(t * 1e6, 2), "weight_GBps": round(wbytes / t / 1e9, 1)}


def decode_dense_leg(S, torch, D, steps, warmup):
    """Comparator: the same decode stream on dense ternary weights (every position a 2-bit code,
    no mask: the BitNet b1.58 layer without Sparse-BitNet's N:M, BL_LAYOUT_DENSE2 with N = M = 4),
    same activations and launch structure.  Both formats move 0.25 B per dense weight."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1000)                              # the decode masters, drawn in the same order
    mats = []
    for i in range(N_PAIRS):
        for (n, K) in (UP, DOWN):
            W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02)
            codes, _, gamma = S.pack(W.contiguous(), 4, 4, S.BL_LAYOUT_DENSE2)
            del W
            mats.append((n, K, codes, gamma))
    packed = sum(c.numel() for (_, _, c, _) in mats)
    groups = {}
    for T in DECODE_T:
        projs = []
        for i, (n, K, codes, gamma) in enumerate(mats):
            xq, sc = D.q[(T, K)]
            j = i // 2
            projs.append(dict(xq=xq[j * T:(j + 1) * T], scale=sc[j * T:(j + 1) * T], K=K,
                              codes=codes, meta=None, gamma=gamma, n=n,
                              y=torch.empty((T, n), dtype=torch.float32, device="cuda")))
        groups[T] = S.FwdGroup(projs, 4, 4, S.BL_LAYOUT_DENSE2)

    def step():
        for T in DECODE_T:
            D.quantize(S, T)
            groups[T]()

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    dense_weights = sum(n * K for (n, K, _, _) in mats)
    return {"workload": "the decode stream (64 up/down pairs, T = 1, 4, 16) on dense ternary "
                        "weights: 2-bit codes at every position, no N:M mask (4:4, dense 2-bit "
                        "layout), same activations and grouped launches",
            "ms_per_step": round(ms, 4), "packed_bytes_per_pass": packed,
            "weight_GBps": round(packed * len(DECODE_T) / (ms * 1e-3) / 1e9, 1),
            "dense_weights_per_s": float(f"{dense_weights * len(DECODE_T) / (ms * 1e-3):.4g}"),
            "vs_sparse_2of4_step": round(ms / D.last_graph_ms_per_step, 3) if D.last_graph_ms_per_step else None}


def _sparse6_groups(S, torch, D):
    """The decode masters re-encoded as SPARSE6 streams and one SPARSE6 group per T over the
    decode workload's quantized activations."""
    mats6 = [(n, K, S.transcode6(codes, meta, n, K), gamma)
             for (n, K, codes, meta, gamma) in D.mats]
    groups, ys = {}, {}
    for T in DECODE_T:
        projs = []
        for i, (n, K, st, gamma) in enumerate(mats6):
            xq, sc = D.q[(T, K)]
            j = i // 2
            projs.append(dict(xq=xq[j * T:(j + 1) * T], scale=sc[j * T:(j + 1) * T], K=K,
                              codes=st, meta=None, gamma=gamma, n=n,
                              y=torch.empty((T, n), dtype=torch.float32, device="cuda")))
        ys[T] = [p["y"] for p in projs]
        groups[T] = S.FwdGroup(projs, 2, 4, S.BL_LAYOUT_SPARSE6)
    return mats6, groups, ys


def decode_sparse6_leg(S, torch, D, ref, steps, warmup):
    """The decode stream on SPARSE6 weights: the 128 packed 2:4 masters re-encoded at 6 bits per
    4-wide group (0.1875 B per weight against 0.25), same activations and grouped launches.
    Checked bitwise against the 2:4 step's outputs, graph-captured and timed like the main metric;
    the group launch of each T is also timed with events beside the 2:4 group's."""
    mats6, groups, ys = _sparse6_groups(S, torch, D)
    stream_bytes = sum(st.numel() for (_, _, st, _) in mats6)

    def step(events=None):
        for T in DECODE_T:
            D.quantize(S, T)
            if events is not None:
                events[T][0].record()
            groups[T]()
            if events is not None:
                events[T][1].record()

    step()
    torch.cuda.synchronize()
    for T in DECODE_T:
        for y, r in zip(ys[T], ref[T]):
            if not torch.equal(y, r):
                raise RuntimeError("SPARSE6 decode differs from the 2:4 decode")
    ms = _graph_ms(torch, step, steps, warmup)
    per_T = {T: [] for T in DECODE_T}
    per_T4 = {T: [] for T in DECODE_T}
    for _ in range(max(1, min(steps, 10))):
        ev = {T: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for T in DECODE_T}
        ev4 = {T: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for T in DECODE_T}
        step(ev)
        D.step(S, ev4)
        torch.cuda.synchronize()
        for T in DECODE_T:
            per_T[T].append(ev[T][0].elapsed_time(ev[T][1]) * 1e-3)
            per_T4[T].append(ev4[T][0].elapsed_time(ev4[T][1]) * 1e-3)
    algo = {T: sum(st.numel() + T * K + 4 * T + 4 * T * n + 4 for (n, K, st, _) in mats6)
            for T in DECODE_T}
    t6 = {T: float(np.mean(per_T[T])) for T in DECODE_T}
    t4 = {T: float(np.mean(per_T4[T])) for T in DECODE_T}
    achieved = sum(algo.values()) / sum(t6.values()) / 1e9
    dense_weights = sum(n * K for (n, K, _, _) in mats6)
    return {"workload": "the decode stream (64 up/down pairs, T = 1, 4, 16) on SPARSE6 weights: the "
                        "2:4 masters re-encoded at 6 bits per group, same activations and grouped "
                        "launches",
            "ms_per_step": round(ms, 4), "stream_bytes_per_pass": stream_bytes,
            "packed_2of4_bytes_per_pass": D.packed_bytes,
            "weight_GBps": round(stream_bytes * len(DECODE_T) / (ms * 1e-3) / 1e9, 1),
            "dense_weights_per_s": float(f"{dense_weights * len(DECODE_T) / (ms * 1e-3):.4g}"),
            "vs_sparse_2of4_step": round(ms / D.last_graph_ms_per_step, 3) if D.last_graph_ms_per_step else None,
            "outputs_identical_to_2of4": True,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "kernel": "gemv6_group_kernel",
                         "per_T": {str(T): {"launch_us": round(t6[T] * 1e6, 2),
                                            "launch_us_2of4": round(t4[T] * 1e6, 2),
                                            "speedup_vs_2of4": round(t4[T] / t6[T], 3),
                                            "algorithmic_bytes": algo[T],
                                            "GBps": round(algo[T] / t6[T] / 1e9, 1)}
                                   for T in DECODE_T}}}


def decode_hybrid_leg(S, torch, D, steps, warmup, dense_frac=0.25):
    """Comparator in the manner of Spense's hybrid format: each projection keeps a quarter of its
    output rows dense (4:4 dense 2-bit codes) and the rest 2:4, as two grouped launches per T (one
    per layout) over the same activations.  Both regions move 0.25 B per dense weight."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1000)                              # the decode masters, drawn in the same order
    sp, dn = [], []
    for i in range(N_PAIRS):
        for (n, K) in (UP, DOWN):
            W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02)
            r = int(round(n * dense_frac / 32)) * 32
            c, _, ga = S.pack(W[:r].contiguous(), 4, 4, S.BL_LAYOUT_DENSE2)
            dn.append((i, r, K, c, None, ga))
            c, m, ga = S.pack(W[r:].contiguous(), 2, 4)
            sp.append((i, n - r, K, c, m, ga))
            del W
    packed = sum(c.numel() + (m.numel() if m is not None else 0)
                 for part in (sp, dn) for (_, _, _, c, m, _) in part)
    groups = {}
    for T in DECODE_T:
        per_layout = []
        for part, (N, M, layout) in ((sp, (2, 4, S.BL_LAYOUT_SPARSE)),
                                     (dn, (4, 4, S.BL_LAYOUT_DENSE2))):
            projs = []
            for (i, n, K, c, m, ga) in part:
                xq, sc = D.q[(T, K)]
                j = i // 2
                projs.append(dict(xq=xq[j * T:(j + 1) * T], scale=sc[j * T:(j + 1) * T], K=K,
                                  codes=c, meta=m, gamma=ga, n=n,
                                  y=torch.empty((T, n), dtype=torch.float32, device="cuda")))
            per_layout.append(S.FwdGroup(projs, N, M, layout))
        groups[T] = per_layout

    def step():
        for T in DECODE_T:
            D.quantize(S, T)
            for grp in groups[T]:
                grp()

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        step()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    return {"workload": "the decode stream (64 up/down pairs, T = 1, 4, 16) with the first quarter "
                        "of every projection's output rows dense ternary (4:4 dense 2-bit codes) "
                        "and the rest 2:4: two grouped launches per T",
            "ms_per_step": round(ms, 4), "packed_bytes_per_pass": packed,
            "weight_GBps": round(packed * len(DECODE_T) / (ms * 1e-3) / 1e9, 1),
            "vs_sparse_2of4_step": round(ms / D.last_graph_ms_per_step, 3) if D.last_graph_ms_per_step else None}


def kernel_source_sha():
    h = hashlib.sha256()
    for f in GROUP_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per grouped-GEMV launch (mean over the T = 1, 4, 16 launches) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    if not os.path.exists(PROFILE_PMC):
        return None
    txt = open(PROFILE_PMC).read()
    m_sha = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.]+)", txt)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


# ---------------------------------------------------------------------------------------------
# prefill leg
# ---------------------------------------------------------------------------------------------

def prefill_leg(S, torch, iters=10):
    from synth import act_student_t, rng, to_bf16
    n, K, T = 11008, 4096, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).contiguous()
    codes, meta, gamma = S.pack(W, 2, 4)
    del W
    x, bits = to_bf16(act_student_t(rng(3), T, K))
    xb = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    xq, sc = S.act_quant(xb)
    y = torch.empty((T, n), dtype=torch.float32, device="cuda")
    L = S.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        L.bitlinear_fwd(xq.data_ptr(), sc.data_ptr(), T, K, codes.data_ptr(), meta.data_ptr(),
                        gamma.data_ptr(), 2, 4, 0, n, y.data_ptr(), None, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        st = L.bitlinear_fwd(xq.data_ptr(), sc.data_ptr(), T, K, codes.data_ptr(), meta.data_ptr(),
                             gamma.data_ptr(), 2, 4, 0, n, y.data_ptr(), None, stream)
        b.record()
        assert st == 0
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    ops = 2.0 * T * K * n
    tops = ops / (ms * 1e-3) / 1e12
    return {"workload": "prefill 4096 tokens x 4096 -> 11008, 2:4, Student-t(4)*0.5 bf16 activations",
            "metric": "prefill dense-equiv int8 TOPS", "value": round(tops, 1), "unit": "TOPS",
            "gemm_ms": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tops, 1), "peak": SMFMAC_I8_PEAK_TOPS,
                         "unit": "TOPS", "frac": round(tops / SMFMAC_I8_PEAK_TOPS, 4), "traffic": None}}


def _event_ms(torch, fn, iters):
    """Mean duration of fn() over iters launches (after three warm-up calls), HIP events on the
    launch stream."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def windows_leg(S, torch, N, M, iters=10, K=4096):
    """(M-2):M through M/2 - 1 overlapping 2:4 windows (lifted activations, sparse MFMA) against
    the dense-stored path of the same masked ternary weights (dense MFMA): 2048 x K -> 4096."""
    n, T = 4096, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(68 if M == 8 else 1416 if M == 16 else 1000 + M)
    W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).contiguous()
    cs, ms, gs = S.pack(W, N, M, S.BL_LAYOUT_SPARSE)
    cd, _, gd = S.pack(W, N, M, S.BL_LAYOUT_DENSE2)
    del W
    x = torch.randn((T, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    xl, sl = S.act_quant(x, M)
    xd, sd = S.act_quant(x, 0)
    ys = torch.empty((T, n), dtype=torch.float32, device="cuda")
    yd = torch.empty((T, n), dtype=torch.float32, device="cuda")
    t_s = _event_ms(torch, lambda: S.fwd(xl, sl, K, cs, ms, gs, n, N, M, S.BL_LAYOUT_SPARSE,
                                         out=(ys, None)), iters)
    t_d = _event_ms(torch, lambda: S.fwd(xd, sd, K, cd, None, gd, n, N, M, S.BL_LAYOUT_DENSE2,
                                         out=(yd, None)), iters)
    t_ql = _event_ms(torch, lambda: S.act_quant(x, M, out=(xl, sl)), iters)
    t_qd = _event_ms(torch, lambda: S.act_quant(x, 0, out=(xd, sd)), iters)
    torch.cuda.synchronize()
    same = bool(torch.equal(ys, yd))   # same masked ternary product, bit for bit, at full size
    if not same:
        raise RuntimeError(f"{N}:{M} window path and dense path disagree")
    ops = 2.0 * T * K * n
    windows = M // 2 - 1
    return {"workload": f"{N}:{M} as {windows} overlapping 2:4 windows, 2048 tokens x {K} -> 4096, "
                        "N(0,1) bf16",
            "windows_TOPS": round(ops / (t_s * 1e-3) / 1e12, 1),
            "dense_TOPS": round(ops / (t_d * 1e-3) / 1e12, 1),
            "gemm_ms": {"windows": round(t_s, 4), "dense": round(t_d, 4)},
            "act_quant_ms": {"lifted": round(t_ql, 4), "plain": round(t_qd, 4)},
            "roofline": {"windows": {"bound": "mfma", "peak": SMFMAC_I8_PEAK_TOPS, "unit": "TOPS",
                                     "frac": round(ops / (t_s * 1e-3) / 1e12 / SMFMAC_I8_PEAK_TOPS, 4)},
                         "dense": {"bound": "mfma", "peak": MFMA_I8_PEAK_TOPS, "unit": "TOPS",
                                   "frac": round(ops / (t_d * 1e-3) / 1e12 / MFMA_I8_PEAK_TOPS, 4)}},
            "speedup_vs_dense": round(t_d / t_s, 3),
            "speedup_with_quant": round((t_d + t_qd) / (t_s + t_ql), 3),
            "bound": round((M // 2) / (M // 2 - 1), 3),
            "outputs_identical": same}


TRAIN_LAYERS = (("q", 3200, 3200), ("k", 3200, 3200), ("v", 3200, 3200), ("o", 3200, 3200),
                ("gate", 8640, 3200), ("up", 8640, 3200), ("down", 3200, 8640))


def train_step_leg(S, torch, iters=3):
    """3B-alike decoder layer set at 8192 tokens: re-mask + ternarize + pack all 7 fp32 masters
    (one grouped pack), quantize the two activation matrices once (one grouped act_quant), the 7
    2:4 forwards (one grouped prefill launch), then the grouped backward of all 7.  Each phase is
    timed with events around its stream launches, and as a HIP graph replay beside them (graphs
    checked against the eager run of the separate calls); the separate pack, act_quant, forward
    and backward calls are timed beside the grouped ones."""
    T = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(35)
    masters, packed, ys = [], [], []
    for (_, n, K) in TRAIN_LAYERS:
        W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).contiguous()
        masters.append(W)
        packed.append(S.pack(W, 2, 4))
        ys.append(torch.empty((T, n), dtype=torch.float32, device="cuda"))
    ws = torch.empty(max(S.packed_bytes(n, K)[3] for (_, n, K) in TRAIN_LAYERS),
                     dtype=torch.uint8, device="cuda")
    X = {K: torch.randn((T, K), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
         for K in (3200, 8640)}
    Q = {K: S.act_quant(X[K]) for K in X}
    # backward operands: output gradients dY (bf16 N(0, 2^-20)), the weight gradients of every
    # master, and one input gradient per activation matrix, summed over the projections reading it
    dYs = [(torch.randn((T, n), generator=g, device="cuda", dtype=torch.float32) * 2.0 ** -10)
           .to(torch.bfloat16) for (_, n, K) in TRAIN_LAYERS]
    dWs = [torch.empty((n, K), dtype=torch.float32, device="cuda") for (_, n, K) in TRAIN_LAYERS]
    dXs = {K: torch.empty((T, K), dtype=torch.float32, device="cuda") for K in X}
    bws = torch.empty(max(S.bwd_workspace_bytes(T, n, K) for (_, n, K) in TRAIN_LAYERS),
                      dtype=torch.uint8, device="cuda")

    def pack_seq():
        for W, out in zip(masters, packed):
            S.pack(W, 2, 4, out=out, ws=ws)

    # the same seven packs as one grouped pack (each of the pack's launches once for all seven)
    pgroup = S.PackGroup([dict(W=W, out=p) for W, p in zip(masters, packed)])

    def pack_all():
        pgroup()

    def quant_seq():
        for K in X:
            S.act_quant(X[K], out=Q[K])

    def quant_all():
        S.act_quant_group([X[K] for K in X], outs=[Q[K] for K in X])

    def fwd_seq():
        for (_, n, K), (c, m, ga), y in zip(TRAIN_LAYERS, packed, ys):
            xq, sc = Q[K]
            S.fwd(xq, sc, K, c, m, ga, n, out=(y, None))

    # the same seven forwards as one grouped prefill launch
    fgroup = S.GemmGroup([dict(xq=Q[K][0], scale=Q[K][1], K=K, codes=c, meta=m, gamma=ga, n=n, y=y)
                          for (_, n, K), (c, m, ga), y in zip(TRAIN_LAYERS, packed, ys)])

    def fwd_all():
        fgroup()

    def bwd_seq():
        seen = set()
        for (_, n, K), (c, m, ga), dy, dw in zip(TRAIN_LAYERS, packed, dYs, dWs):
            xq, sc = Q[K]
            S.bwd(dy, xq, sc, K, c, m, ga, n, out=(dXs[K], dw), accumulate=(K in seen, False),
                  ws=bws)
            seen.add(K)

    # the same seven calls as one grouped backward (one operand launch, one product launch)
    projs, seen = [], set()
    for (_, n, K), (c, m, ga), dy, dw in zip(TRAIN_LAYERS, packed, dYs, dWs):
        xq, sc = Q[K]
        projs.append(dict(dy=dy, xq=xq, scale=sc, K=K, codes=c, meta=m, gamma=ga, n=n,
                          dx=dXs[K], dw=dw, accumulate=(K in seen, False)))
        seen.add(K)
    bgroup = S.BwdGroup(projs, T)

    def bwd_all():
        bgroup()

    # each phase also captured as a HIP graph; two replays are checked bitwise against the eager
    # results first
    def results():
        return ([t for (c, m, ga) in packed for t in (c, m, ga)] + [t for K in Q for t in Q[K]] +
                ys + dWs + list(dXs.values()))

    def outputs():
        return [t.clone() for t in results()]

    pack_seq()
    quant_seq()
    fwd_seq()
    bwd_seq()
    torch.cuda.synchronize()
    ref = outputs()
    for t in results():
        t.zero_()
    pack_all()
    quant_all()
    fwd_all()
    bwd_all()
    torch.cuda.synchronize()
    for a, b in zip(outputs(), ref):
        if not torch.equal(a, b):
            raise RuntimeError("grouped pack, act_quant, forward or backward differs from the sequential calls")
    graphs = []
    cap = torch.cuda.Stream()
    for fn in (pack_seq, pack_all, quant_seq, quant_all, fwd_seq, fwd_all, bwd_seq, bwd_all):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr, stream=cap):
            fn()
        graphs.append(gr)
    for _ in range(2):
        for t in results():
            t.zero_()
        for gr in graphs:
            gr.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(), ref):
            if not torch.equal(a, b):
                raise RuntimeError("training-step graph replay differs from the eager run")
    # every phase timed as stream launches (the figures below) and as its graph's replay (beside
    # them, graph_ms): each kernel node of a replayed graph starts later than the same launch on
    # the stream, which shows most in the phases made of several short launches
    fns = (pack_seq, pack_all, quant_seq, quant_all, fwd_seq, fwd_all, bwd_seq, bwd_all)
    t_graph = [_event_ms(torch, gr.replay, iters) for gr in graphs]
    (t_pack_seq, t_pack, t_quant_seq, t_quant, t_fwd_seq, t_fwd, t_bwd_seq,
     t_bwd) = [_event_ms(torch, fn, iters) for fn in fns]
    torch.cuda.synchronize()
    for a, b in zip(outputs(), ref):
        if not torch.equal(a, b):
            raise RuntimeError("training-step timed launches differ from the first eager run")
    pack_bytes = sum(4 * n * K + p[0].numel() + p[1].numel() for (_, n, K), p in zip(TRAIN_LAYERS, packed))
    # act_quant: bf16 read + int8 write per element + 4 B scale per token
    quant_bytes = sum(T * K * 3 + 4 * T for K in X)
    ops = sum(2.0 * T * K * n for (_, n, K) in TRAIN_LAYERS)
    pack_gbs = pack_bytes / (t_pack * 1e-3) / 1e9
    quant_gbs = quant_bytes / (t_quant * 1e-3) / 1e9
    fwd_tops = ops / (t_fwd * 1e-3) / 1e12
    # backward: two dense bf16 products (dX and dW) of 2 T K n flops each per projection
    bwd_tflops = 2 * ops / (t_bwd * 1e-3) / 1e12
    return {"workload": "3B-alike layer set (QKV 3x3200x3200, O, gate/up 8640x3200, down 3200x8640), "
                        "8192 tokens, 2:4, bf16 N(0,1) activations, bf16 output gradients",
            "step_ms": round(t_pack + t_quant + t_fwd + t_bwd, 4),
            "bwd_ms": round(t_bwd, 4), "bwd_TFLOPS": round(bwd_tflops, 1),
            # the seven bitlinear_bwd calls one after another (same results, bit for bit)
            "bwd_sequential_ms": round(t_bwd_seq, 4),
            "pack_ms": round(t_pack, 4), "pack_GBps": round(pack_gbs, 1),
            # the seven bitlinear_pack calls one after another (same results, bit for bit)
            "pack_sequential_ms": round(t_pack_seq, 4),
            "act_quant_ms": round(t_quant, 4), "act_quant_GBps": round(quant_gbs, 1),
            # the two act_quant_i8 calls one after another (same results, bit for bit)
            "act_quant_sequential_ms": round(t_quant_seq, 4),
            "fwd_ms": round(t_fwd, 4), "fwd_TOPS": round(fwd_tops, 1),
            # the seven bitlinear_fwd calls one after another (same results, bit for bit)
            "fwd_sequential_ms": round(t_fwd_seq, 4),
            "graph_ms": {k: round(v, 4) for k, v in zip(
                ("pack_sequential", "pack", "act_quant_sequential", "act_quant", "fwd_sequential",
                 "fwd", "bwd_sequential", "bwd"), t_graph)},
            # algorithmic bytes (pack: 4 B read + packed bytes written per weight, one pass over
            # the master; act_quant: 3 B per element + 4 B per token) or dense-equivalent ops
            "roofline": {"pack": {"bound": "hbm", "achieved": round(pack_gbs, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(pack_gbs / HBM_PEAK_GBS, 4)},
                         "act_quant": {"bound": "hbm", "achieved": round(quant_gbs, 1),
                                       "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": round(quant_gbs / HBM_PEAK_GBS, 4)},
                         "fwd": {"bound": "mfma", "achieved": round(fwd_tops, 1),
                                 "peak": SMFMAC_I8_PEAK_TOPS, "unit": "TOPS",
                                 "frac": round(fwd_tops / SMFMAC_I8_PEAK_TOPS, 4)},
                         "bwd": {"bound": "mfma", "achieved": round(bwd_tflops, 1),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(bwd_tflops / BF16_PEAK_TFLOPS, 4)}}}


def bwd_profile_pass(S, torch):
    """Backward of one training-step projection (gate, 8640 x 3200, 8192 tokens), three times."""
    T, n, K = 8192, 8640, 3200
    g = torch.Generator(device="cuda")
    g.manual_seed(36)
    W = (torch.randn((n, K), generator=g, device="cuda") * 0.02).contiguous()
    codes, meta, gamma = S.pack(W, 2, 4)
    x = torch.randn((T, K), generator=g, device="cuda").to(torch.bfloat16)
    xq, sc = S.act_quant(x)
    dy = (torch.randn((T, n), generator=g, device="cuda") * 2.0 ** -10).to(torch.bfloat16)
    dx = torch.empty((T, K), device="cuda")
    dw = torch.empty((n, K), device="cuda")
    ws = torch.empty(S.bwd_workspace_bytes(T, n, K), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        S.bwd(dy, xq, sc, K, codes, meta, gamma, n, out=(dx, dw), ws=ws)


def bwd_group_profile_pass(S, torch):
    """Grouped backward of the training-step layer set (8192 tokens) three times, then two plain
    device copies of COPY_BYTES (the counters' scale reference)."""
    T = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(37)
    X = {K: S.act_quant(torch.randn((T, K), generator=g, device="cuda").to(torch.bfloat16))
         for K in (3200, 8640)}
    dXs = {K: torch.empty((T, K), device="cuda") for K in X}
    projs, seen = [], set()
    for (_, n, K) in TRAIN_LAYERS:
        W = (torch.randn((n, K), generator=g, device="cuda") * 0.02).contiguous()
        c, m, ga = S.pack(W, 2, 4)
        dy = (torch.randn((T, n), generator=g, device="cuda") * 2.0 ** -10).to(torch.bfloat16)
        projs.append(dict(dy=dy, xq=X[K][0], scale=X[K][1], K=K, codes=c, meta=m, gamma=ga, n=n,
                          dx=dXs[K], dw=torch.empty((n, K), device="cuda"),
                          accumulate=(K in seen, False)))
        seen.add(K)
    grp = S.BwdGroup(projs, T)
    for _ in range(3):
        grp()
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)


def fwd_group_profile_pass(S, torch):
    """Forward of the training-step layer set (8192 tokens, 2:4): the grouped prefill launch three
    times, then the seven separate bitlinear_fwd calls three times, then two plain device copies
    of COPY_BYTES (the counters' scale reference)."""
    T = 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(38)
    X = {K: S.act_quant(torch.randn((T, K), generator=g, device="cuda").to(torch.bfloat16))
         for K in (3200, 8640)}
    projs = []
    for (_, n, K) in TRAIN_LAYERS:
        W = (torch.randn((n, K), generator=g, device="cuda") * 0.02).contiguous()
        c, m, ga = S.pack(W, 2, 4)
        projs.append(dict(xq=X[K][0], scale=X[K][1], K=K, codes=c, meta=m, gamma=ga, n=n,
                          y=torch.empty((T, n), device="cuda")))
    grp = S.GemmGroup(projs)
    for _ in range(3):
        grp()
    for _ in range(3):
        for p in projs:
            S.fwd(p["xq"], p["scale"], p["K"], p["codes"], p["meta"], p["gamma"], p["n"],
                  out=(p["y"], None))
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)


# ---------------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the decode workload)
# ---------------------------------------------------------------------------------------------

def _host_description():
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


_CPU_STATE = {}


def _cpu_worker_init():
    """Pack the up/down masters with the oracle in this worker (same seeds as the parent)."""
    import oracle as O
    from synth import master_weights, rng
    g = rng(0)
    Wu, Wd = master_weights(g, *UP), master_weights(g, *DOWN)
    _CPU_STATE["p"] = (O.pack(Wu, 2, 4), O.pack(Wd, 2, 4))


def _cpu_worker_rows(task):
    """Rows r0:r1 of matrix `which`: int64 GEMV of the packed oracle weights + fp64 rescale."""
    import oracle as O
    which, r0, r1, q, s = task
    p = _CPU_STATE["p"][which]
    acc = O.acc_dense(p["W_eff"][r0:r1], q)
    O.rescale(acc, p["gamma"], s)
    return r1 - r0


def cpu_baseline(budget_s):
    """The oracle on a bounded sample of the decode workload (act_quant + int64 GEMV + rescale of
    the up/down pair at T = 1, 4, 16): first one thread, then every usable host core (output rows
    split over a process pool; numpy's int64 matmul runs on one thread).  Runs in a process that
    never touches the GPU."""
    import multiprocessing as mp

    import oracle as O
    from synth import act_normal, rng, to_bf16
    t_pack = time.perf_counter()
    _cpu_worker_init()                                       # the oracle pack of both masters
    t_pack = time.perf_counter() - t_pack
    pu, pd = _CPU_STATE["p"]
    g = rng(0)
    from synth import master_weights
    master_weights(g, *UP), master_weights(g, *DOWN)          # the draws the masters took
    xu, _ = to_bf16(act_normal(g, max(DECODE_T), UP[1]))
    xd, _ = to_bf16(act_normal(g, max(DECODE_T), DOWN[1]))
    packed = 2 * UP[0] * UP[1] // 4
    # one thread (the quantization and the GEMV + rescale also timed apart: the stages)
    done_bytes, n_mats, t0 = 0, 0, time.perf_counter()
    t_q = t_g = 0.0
    q_bytes = 0
    while True:
        for T in DECODE_T:
            for p, x in ((pu, xu), (pd, xd)):
                ta = time.perf_counter()
                q, s = O.act_quant(x[:T])
                tb = time.perf_counter()
                O.rescale(O.acc_dense(p["W_eff"], q), p["gamma"], s)
                tc = time.perf_counter()
                t_q += tb - ta
                t_g += tc - tb
                q_bytes += 3 * q.size + 4 * T          # bf16 read, int8 written, token scales
                done_bytes += packed
                n_mats += 1
        if time.perf_counter() - t0 > budget_s / 2:
            break
    dt1 = time.perf_counter() - t0
    single = done_bytes / dt1 / 1e9
    # every usable core: rows of each matrix split over the workers
    cores = max(1, min(len(os.sched_getaffinity(0)), 64))
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_worker_rows, [(0, 0, 1, np.zeros((1, UP[1]), np.int8), np.ones(1, np.float32))] * cores)
        done_m, n_m, t0 = 0, 0, time.perf_counter()
        while True:
            for T in DECODE_T:
                for which, (p, x) in enumerate(((pu, xu), (pd, xd))):
                    q, s = O.act_quant(x[:T])
                    n = p["W_eff"].shape[0]
                    step = (n + cores - 1) // cores
                    pool.map(_cpu_worker_rows, [(which, r, min(n, r + step), q, s)
                                                for r in range(0, n, step)])
                    done_m += packed
                    n_m += 1
            if time.perf_counter() - t0 > budget_s / 2:
                break
        dtm = time.perf_counter() - t0
    multi = done_m / dtm / 1e9
    pack_bytes = 4 * (UP[0] * UP[1] + DOWN[0] * DOWN[1]) + 2 * packed   # masters read, codes+meta
    return {"value": round(multi, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "single_thread_value": round(single, 4),
            "stages_single_thread": {
                "pack": {"GBps": round(pack_bytes / t_pack / 1e9, 4), "s": round(t_pack, 2),
                         "work": "the up and down masters (35.4 M weights): mask, exact gamma, "
                                 "ternarize, 2:4 pack; 4 B read + 0.25 B written per weight"},
                "act_quant": {"GBps": round(q_bytes / t_q / 1e9, 4), "s": round(t_q, 4),
                              "work": f"{n_mats} token blocks (T = 1, 4, 16), bf16 in, int8 out"},
                "gemv": {"GBps": round(done_bytes / t_g / 1e9, 4), "s": round(t_g, 2),
                         "work": f"{n_mats} int64 GEMVs + fp64 rescales, packed bytes per s"}},
            "host": _host_description(),
            "sample": f"decode up/down pair at T=1,4,16 (act_quant + int64 GEMV + fp64 rescale per "
                      f"matrix pass): {n_mats} passes on one thread in {dt1:.1f} s, then {n_m} "
                      f"passes with the output rows split over {cores} worker processes in "
                      f"{dtm:.1f} s"}


def cpu_baseline_child(budget_s):
    """Run cpu_baseline in a child process that never initializes the GPU; returns its dict."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                        "--cpu-budget-s", str(budget_s)], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"cpu baseline child failed ({r.returncode}): {r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


# ---------------------------------------------------------------------------------------------

def main():
    args = parse()
    if args.cpu_baseline_only:
        print(json.dumps(cpu_baseline(args.cpu_budget_s)), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sparse ternary "
              "BitLinear path is built and measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparsity_amd as S
    S.lib()
    torch.cuda.set_device(0)
    if args.profile_pass == "bwd":
        bwd_profile_pass(S, torch)
        torch.cuda.synchronize()
        log("profile pass done: backward of the gate projection x 3")
        return
    if args.profile_pass == "bwdgroup":
        bwd_group_profile_pass(S, torch)
        torch.cuda.synchronize()
        log("profile pass done: grouped backward of the layer set x 3, copies x 2")
        return
    if args.profile_pass == "fwdgroup":
        fwd_group_profile_pass(S, torch)
        torch.cuda.synchronize()
        log("profile pass done: grouped forward of the layer set x 3, separate calls x 3, copies x 2")
        return
    if args.profile_pass == "train":
        train_step_leg(S, torch, iters=2)
        torch.cuda.synchronize()
        log("profile pass done: training-step layer set")
        return
    if args.profile_pass == "windows":
        windows_leg(S, torch, 6, 8, iters=2)
        torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("profile pass done: 6:8 window and dense GEMMs, 2 copies")
        return
    if args.profile_pass == "prefill":
        prefill_leg(S, torch, iters=2)
        torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("profile pass done: prefill GEMM x 5, 2 copies")
        return
    log(f"device {torch.cuda.get_device_name(0)}; packing {2 * N_PAIRS} matrices")
    D = Decode(S, torch)
    if args.profile_pass == "decode":
        for _ in range(2):
            D.step(S)
        torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"profile pass done: 2 decode steps, 2 copies of {COPY_BYTES} bytes")
        return
    if args.profile_pass == "chain":
        layers = [dict(codes=c, meta=m, gamma=ga, n=n, K=K) for (n, K, c, m, ga) in D.mats]
        for T in DECODE_T:
            ch = S.Chain(layers, T)
            for _ in range(2):
                ch(D.x[(T, UP[1])][:T])
            if ch.error():
                raise RuntimeError("chain launch reported a barrier timeout")
        log("profile pass done: 2 chain launches of the 128 decode layers at T = 1, 4, 16")
        return
    if args.profile_pass == "sparse6":
        _, groups6, _ = _sparse6_groups(S, torch, D)
        for _ in range(2):
            for T in DECODE_T:
                D.quantize(S, T)
                groups6[T]()
                D.groups[T]()
        torch.cuda.synchronize()
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"profile pass done: 2 x (SPARSE6 and 2:4 groups at T = 1, 4, 16), 2 copies")
        return

    # eager reference output of one step, then graph capture of the same step
    D.step(S)
    torch.cuda.synchronize()
    ref = {T: [y.clone() for y in D.ys[T]] for T in DECODE_T}
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        D.step(S)
    for _ in range(2):
        for T in DECODE_T:
            for y in D.ys[T]:
                y.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for T in DECODE_T:
            for y, r in zip(D.ys[T], ref[T]):
                if not torch.equal(y, r):
                    raise RuntimeError("graph replay differs from the eager run")
    log("graph replays match the eager run")

    # The timed steps are stream launches (six per step); the captured graph of the same step is
    # timed beside them.  Each kernel node of a replayed graph starts measurably later than the
    # same kernel launched on the stream, so the graph step is the slower one here.
    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.steps

    graph_ms_per_step = timed(graph.replay)
    ms_per_step = timed(lambda: D.step(S))
    for T in DECODE_T:
        for y, r in zip(D.ys[T], ref[T]):
            if not torch.equal(y, r):
                raise RuntimeError("the timed steps' outputs differ from the eager run")
    value = D.packed_bytes * len(DECODE_T) / (ms_per_step * 1e-3) / 1e9
    log(f"decode step {ms_per_step:.3f} ms -> {value:.1f} GB/s of packed weights "
        f"(graph replay {graph_ms_per_step:.3f} ms)")
    D.last_ms_per_step = ms_per_step
    D.last_graph_ms_per_step = graph_ms_per_step

    # grouped-GEMV launch durations in isolation: HIP events on the launch stream around every
    # grouped launch of eager steps (each measurement also holds the events' own dispatch
    # overhead, several microseconds)
    per_T = {T: [] for T in DECODE_T}
    for _ in range(max(1, min(args.steps, 10))):
        events = {T: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for T in DECODE_T}
        D.step(S, events)
        torch.cuda.synchronize()
        for T in DECODE_T:
            per_T[T].append(events[T][0].elapsed_time(events[T][1]) * 1e-3)
    iso_t = {T: float(np.mean(per_T[T])) for T in DECODE_T}
    algo = {T: D.algorithmic_bytes(T) for T in DECODE_T}

    # layer stream: the grouped launch repeated back to back on already quantized activations
    # (the steady state of a long decode, and how the launches run inside the timed graph), HIP
    # events on the launch stream around LAYER_STREAM_LAUNCHES launches: the mean launch duration
    layer_stream, mean_t = {}, {}
    for T in DECODE_T:
        for _ in range(3):
            D.groups[T]()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(LAYER_STREAM_LAUNCHES):
            D.groups[T]()
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / LAYER_STREAM_LAUNCHES
        mean_t[T] = t
        layer_stream[str(T)] = {"launch_us": round(t * 1e6, 2),
                                "weight_GBps": round(D.packed_bytes / t / 1e9, 1),
                                "algorithmic_GBps": round(algo[T] / t / 1e9, 1),
                                "frac": round(algo[T] / t / 1e9 / HBM_PEAK_GBS, 4)}
    log("layer stream: " + ", ".join(f"T={T} {layer_stream[str(T)]['algorithmic_GBps']} GB/s"
                                     for T in DECODE_T))
    achieved = sum(algo.values()) / sum(mean_t.values()) / 1e9
    traffic = measured_traffic()
    per_T_out = {str(T): {"launch_us": round(mean_t[T] * 1e6, 2),
                          "isolated_launch_us": round(iso_t[T] * 1e6, 2),
                          "algorithmic_bytes": algo[T],
                          "GBps": round(algo[T] / mean_t[T] / 1e9, 1)} for T in DECODE_T}
    log(f"grouped GEMV: " + ", ".join(f"T={T} {mean_t[T] * 1e6:.1f} us (isolated "
                                      f"{iso_t[T] * 1e6:.1f})" for T in DECODE_T) +
        f" -> {achieved:.1f} GB/s algorithmic")

    out = {
        "metric": "decode weight GB/s", "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "graph_ms_per_step": round(graph_ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode GEMV 2:4 ternary, FFN up 6912x2560 + down 2560x6912, "
                               "64 distinct pairs (cold cache), T=1,4,16 bf16 N(0,1); per step and "
                               "T: one grouped act_quant launch of the stacked activations + one "
                               "grouped GEMV launch over the 128 projections, which are "
                               "independent (each reads its own activations; the dependent "
                               "form is the decode_chain leg, one launch per projection the "
                               "decode_single leg)",
                   "tokens": list(DECODE_T), "layer_pairs": N_PAIRS,
                   "packed_weight_bytes_per_pass": D.packed_bytes, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "gemv_group_kernel<SPARSE>",
                     "per_T": per_T_out,
                     "layer_stream": {"launches": LAYER_STREAM_LAUNCHES, "per_T": layer_stream}},
    }
    log("fused decode leg")
    out["decode_fused"] = decode_fused_leg(S, torch, D, ref, args.steps, args.warmup)
    log(f"fused decode {out['decode_fused']['value']} GB/s")
    log("SPARSE6 decode leg")
    out["decode_sparse6"] = decode_sparse6_leg(S, torch, D, ref, args.steps, args.warmup)
    log("sparse6: " + ", ".join(f"T={T} {v['launch_us']} us ({v['speedup_vs_2of4']}x 2:4)"
                                for T, v in out["decode_sparse6"]["roofline"]["per_T"].items()))
    log("single-projection decode leg")
    out["decode_single"] = decode_single_leg(S, torch, D, args.steps, args.warmup)
    log("single: " + ", ".join(f"T={T} {v['weight_GBps']} GB/s" for T, v in out["decode_single"]["per_T"].items()))
    log("dependent chain decode leg")
    out["decode_chain"] = decode_chain_leg(S, torch, D, args.steps, args.warmup)
    log("chain: " + ", ".join(f"T={T} {v['chain_ms']} ms (calls {v['per_layer_calls_ms']} ms)"
                              for T, v in out["decode_chain"]["per_T"].items()))
    if not args.no_extra:
        log("MALL-sized decode reading")
        out["decode_mall_sized"] = decode_mall_leg(S, torch, D)
        log(f"MALL-sized decode {out['decode_mall_sized']['weight_GBps']} GB/s")
        log("dense ternary decode comparator")
        out["decode_dense_ternary"] = decode_dense_leg(S, torch, D, args.steps, args.warmup)
        log(f"dense ternary decode {out['decode_dense_ternary']['ms_per_step']} ms/step")
        log("hybrid dense + 2:4 decode comparator")
        out["decode_hybrid"] = decode_hybrid_leg(S, torch, D, args.steps, args.warmup)
        log(f"hybrid decode {out['decode_hybrid']['ms_per_step']} ms/step")
    if not args.no_prefill:
        log("prefill leg")
        out["prefill"] = prefill_leg(S, torch)
        log(f"prefill {out['prefill']['value']} TOPS")
    if not args.no_extra:
        for key, N, M in (("six_eight", 6, 8), ("fourteen_sixteen", 14, 16)):
            log(f"{N}:{M} leg")
            out[key] = windows_leg(S, torch, N, M)
            log(f"{N}:{M} windows {out[key]['windows_TOPS']} TOPS, dense {out[key]['dense_TOPS']} TOPS")
        # the other (2N-2):2N group sizes, K near 4096 where windows and dense storage both fit
        gen = {}
        for N, M, K in ((4, 6, 3840), (8, 10, 3840), (10, 12, 3840), (12, 14, 3584)):
            r = windows_leg(S, torch, N, M, K=K)
            gen[f"{N}:{M}"] = {k: r[k] for k in ("workload", "windows_TOPS", "dense_TOPS",
                                                 "speedup_vs_dense", "bound", "outputs_identical")}
            log(f"{N}:{M} windows {r['windows_TOPS']} TOPS, dense {r['dense_TOPS']} TOPS")
        out["windows_general"] = gen
        log("training-step layer set leg")
        out["train_step"] = train_step_leg(S, torch)
        log(f"train step {out['train_step']['step_ms']} ms")
    if not args.no_cpu_baseline:
        log("cpu oracle baseline")
        out["cpu_baseline"] = cpu_baseline_child(args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
