#!/usr/bin/env python3
"""Benchmark of the sparse ternary BitLinear forward on one MI355X.

Default workload (decode GEMV, 2:4): FFN up 6912x2560 and down 2560x6912 BitNet-2B-like
projections, 64 distinct up/down pairs (566 MB of packed weights, more than twice the 256 MB
last-level cache, so every step streams them from HBM), bf16 activations ~ N(0,1).  One step is
the decode hot path for the whole layer stream at batch 1, 4 and 16 tokens: per matrix, per-token
int8 quantization of the activations and the sparse ternary GEMV with fused rescale.  Weights are
packed once before timing (inference stores packed weights).  The step is captured once as a HIP
graph and replayed; the graph's output is checked bitwise against an eager run first.

metric: decode weight GB/s = packed weight bytes streamed per step / step time.

Also in the same JSON line:
  roofline      for the GEMV kernel: algorithmic bytes per launch / mean launch duration, the
                durations taken with HIP events on the launch stream around every GEMV launch of
                an eager pass over the same steps; HBM traffic from rocprofv3 counters when the
                committed counter summary matches the current kernel source (else null)
  prefill       4096 x 4096 -> 11008 2:4 GEMM (Student-t activations): dense-equivalent int8 TOPS
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
SMFMAC_I8_PEAK_TOPS = 10100.0  # MI355X int8 with 2:4 structured sparsity, dense-equivalent
UP = (6912, 2560)
DOWN = (2560, 6912)
N_PAIRS = 64
DECODE_T = (1, 4, 16)
PROFILE_PMC = os.path.join(ROOT, "profiles", "gemv_decode_pmc.md")
FWD_SRC = os.path.join(ROOT, "sparsity_amd", "csrc", "fwd.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------------
# decode workload
# ---------------------------------------------------------------------------------------------

class Matrix:
    """One packed projection plus its activation/output buffers, with raw pointers for launches."""

    def __init__(self, S, torch, n, K, seed):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        W = (torch.randn((n, K), generator=g, device="cuda", dtype=torch.float32) * 0.02).contiguous()
        self.n, self.K = n, K
        self.codes, self.meta, self.gamma = S.pack(W, 2, 4)
        del W
        x = torch.randn((max(DECODE_T), K), generator=g, device="cuda", dtype=torch.float32)
        self.x = x.to(torch.bfloat16).contiguous()
        self.packed_bytes = self.codes.numel() + self.meta.numel()


def decode_setup(S, torch):
    mats = []
    for i in range(N_PAIRS):
        mats.append(Matrix(S, torch, *UP, seed=1000 + 2 * i))
        mats.append(Matrix(S, torch, *DOWN, seed=1001 + 2 * i))
    Tm = max(DECODE_T)
    bufs = {}
    for K in (UP[1], DOWN[1]):
        bufs[("xq", K)] = torch.empty((Tm, K), dtype=torch.int8, device="cuda")
        bufs[("sc", K)] = torch.empty(16, dtype=torch.float32, device="cuda")
    for n in (UP[0], DOWN[0]):
        bufs[("y", n)] = torch.empty((Tm, n), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    return mats, bufs


def make_step(S, torch, mats, bufs, events=None):
    L = S.lib()
    aq, fw = L.act_quant_i8, L.bitlinear_fwd
    plan = []
    for T in DECODE_T:
        for m in mats:
            xq, sc, y = bufs[("xq", m.K)], bufs[("sc", m.K)], bufs[("y", m.n)]
            plan.append((T, m.x.data_ptr(), m.K, xq.data_ptr(), sc.data_ptr(), m.codes.data_ptr(),
                         m.meta.data_ptr(), m.gamma.data_ptr(), m.n, y.data_ptr()))

    def step():
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for i, (T, x, K, xq, sc, c, me, ga, n, y) in enumerate(plan):
            st = aq(x, 1, T, K, 0, xq, sc, stream)
            if events is not None:
                events[i][0].record()
            st |= fw(xq, sc, T, K, c, me, ga, 2, 4, 0, n, y, None, stream)
            if events is not None:
                events[i][1].record()
            if st:
                raise RuntimeError(f"launch failed with status {st}")
    return step, plan


def gemv_algorithmic_bytes(T, n, K, packed):
    # codes + meta + int8 activations + fp32 token scales + fp32 outputs + gamma
    return packed + T * K + 4 * T + 4 * T * n + 4


def kernel_source_sha():
    return hashlib.sha256(open(FWD_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per GEMV launch from the committed rocprofv3 counter summary, if current."""
    if not os.path.exists(PROFILE_PMC):
        return None
    txt = open(PROFILE_PMC).read()
    m_sha = re.search(r"fwd_source_sha256_16:\s*([0-9a-f]+)", txt)
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


# ---------------------------------------------------------------------------------------------
# CPU oracle baseline (bounded sample of the decode workload)
# ---------------------------------------------------------------------------------------------

def cpu_baseline(budget_s):
    import oracle as O
    from synth import act_normal, master_weights, rng, to_bf16
    g = rng(0)
    Wu, Wd = master_weights(g, *UP), master_weights(g, *DOWN)
    pu, pd = O.pack(Wu, 2, 4), O.pack(Wd, 2, 4)
    xu, _ = to_bf16(act_normal(g, max(DECODE_T), UP[1]))
    xd, _ = to_bf16(act_normal(g, max(DECODE_T), DOWN[1]))
    packed = 2 * UP[0] * UP[1] // 4
    done_bytes, n_mats, t0 = 0, 0, time.perf_counter()
    while True:
        for T in DECODE_T:
            for p, x in ((pu, xu), (pd, xd)):
                q, s = O.act_quant(x[:T])
                O.rescale(O.acc_dense(p["W_eff"], q), p["gamma"], s)
                done_bytes += packed
                n_mats += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_mats} matrix passes (act_quant + int64 GEMV + rescale) of the up/down pair "
                      f"at T=1,4,16, {dt:.1f} s, numpy single thread"}


# ---------------------------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sparse ternary "
              "BitLinear path is built and measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparsity_amd as S
    S.lib()
    torch.cuda.set_device(0)
    log(f"device {torch.cuda.get_device_name(0)}; packing {2 * N_PAIRS} matrices")
    mats, bufs = decode_setup(S, torch)
    weight_bytes_per_pass = sum(m.packed_bytes for m in mats)
    step, plan = make_step(S, torch, mats, bufs)

    # eager reference output of one step, then graph capture
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in bufs.items() if k[0] == "y"}
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=cap):
        step()
    for k in ref:
        bufs[k].zero_()
    graph.replay()
    torch.cuda.synchronize()
    for k, v in ref.items():
        if not torch.equal(bufs[k], v):
            raise RuntimeError("graph replay differs from the eager run")
    log("graph replay matches eager run")

    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = weight_bytes_per_pass * len(DECODE_T) / (ms_per_step * 1e-3) / 1e9
    log(f"decode step {ms_per_step:.3f} ms -> {value:.1f} GB/s of packed weights")

    # per-launch GEMV durations with events on the launch stream (eager pass over the same steps)
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in plan]
    estep, _ = make_step(S, torch, mats, bufs, events)
    per_T = {T: [] for T in DECODE_T}
    algo = {T: [] for T in DECODE_T}
    for _ in range(max(1, min(args.steps, 5))):
        estep()
        torch.cuda.synchronize()
        for (a, b), p in zip(events, plan):
            T, K, n = p[0], p[2], p[8]
            per_T[T].append(a.elapsed_time(b) * 1e-3)
            algo[T].append(gemv_algorithmic_bytes(T, n, K, mats[0].packed_bytes))
    all_t = [t for T in DECODE_T for t in per_T[T]]
    all_b = [b for T in DECODE_T for b in algo[T]]
    mean_t = float(np.mean(all_t))
    achieved = float(np.mean(all_b)) / mean_t / 1e9
    traffic = measured_traffic()
    per_T_out = {str(T): {"gemv_us": round(float(np.mean(per_T[T])) * 1e6, 3),
                          "gemv_GBps": round(float(np.mean(algo[T])) / float(np.mean(per_T[T])) / 1e9, 1)}
                 for T in DECODE_T}
    log(f"GEMV mean launch {mean_t * 1e6:.2f} us -> {achieved:.1f} GB/s algorithmic")

    out = {
        "metric": "decode weight GB/s", "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "decode GEMV 2:4 ternary, FFN up 6912x2560 + down 2560x6912, "
                               "64 distinct pairs (cold cache), T=1,4,16 bf16 N(0,1)",
                   "tokens": list(DECODE_T), "layer_pairs": N_PAIRS,
                   "packed_weight_bytes_per_pass": weight_bytes_per_pass, "parallelism": "none"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "gemv_kernel<SPARSE>",
                     "mean_launch_us": round(mean_t * 1e6, 3), "per_T": per_T_out},
    }
    if not args.no_prefill:
        log("prefill leg")
        out["prefill"] = prefill_leg(S, torch)
        log(f"prefill {out['prefill']['value']} TOPS")
    if not args.no_cpu_baseline:
        log("cpu oracle baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
