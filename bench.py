"""Benchmark of the grouped 4-bit MoE hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Headline workload (one JSON line on stdout): Qwen3-30B-A3B-shaped NF4
decode at M = 1 token, top-8 of E = 128 experts.  One step is one decode
token through both expert projections: the gate_up GEMV (W [1536, 2048])
and the down GEMV (W [2048, 768], one input row per routed pair).  Every
step has its own routing and reads one of 16 independent copies of each
expert bank in turn, so the active experts' bytes come from HBM and not
from the 256 MB last-level cache.  The K timed steps are captured once in a
HIP graph and replayed (a decode loop's launch pattern), bracketed by
device synchronisation.  ``value`` is algorithmic bytes per second: packed
codes + absmax of the distinct active experts, activations read once,
outputs written once.

The same line carries
  * ``roofline``: the gate_up GEMV kernel's algorithmic bytes per launch over
    its average device time per launch, from HIP events around a replayed
    graph of K gate_up launches on the launch stream, against the 8 TB/s HBM
    peak; plus same-run controls: the empty-launch floor and a plain
    streaming read of the same byte count from cold memory;
  * ``cpu_baseline``: the CPU oracle (decode + float64 grouped matmul) on a
    bounded sample of the same decode steps;
  * ``prefill``: Qwen3 NF4 prefill (M = 4096, Zipf(1.1) top-8, router
    weights) -- route sort + gate_up GEMM + down GEMM -- in TFLOP/s against
    the dense bf16 MFMA peak;
  * ``extra``: MXFP4 gpt-oss-20b decode (M = 1), prefill (M = 2048) and dgrad
    (M = 2048, top-4), NF4 dgrad (M = 2048, top-8), the NF4 M = 4 decode, and
    the whole NF4 MoE layer (SwiGLU and router-weighted combine fused) at
    decode (M = 1) and prefill (M = 4096).
The prefill and dgrad steps run eagerly (their kernels are long): the step
time comes from a loop without any events; the per-kernel times from a
second loop with events around each launch.
All inputs are synthetic and resident in HBM before timing starts.
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bit_grouped_moe_amd as gq  # noqa: E402
import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6        # MI355X dense bf16 MFMA
FP4_PEAK_TFLOPS = 10066.0        # MI355X dense fp4 MFMA
COPIES = 16                      # independent bank copies rotated per step
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def nf4_expert_bytes(N, K):
    return N * K // 2 + N * (K // 64) * 4


def mx_expert_bytes(N, K):
    return N * K // 2 + N * (K // 32)


def bf16_dev(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def capture(fn, n):
    """HIP graph of fn(0) .. fn(n-1) captured on a side stream."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    return g


def event_ms(fn):
    """Device time of fn() from HIP events on the current stream."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


class Timer:
    """Event pairs around individual launches (long kernels only: the queue
    stays busy, so host launch latency does not leak into the pair)."""

    def __init__(self):
        self.pairs = []

    def start(self):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        return ev

    def stop(self, ev0):
        ev1 = torch.cuda.Event(enable_timing=True)
        ev1.record()
        self.pairs.append((ev0, ev1))

    def avg_us(self):
        return 1e3 * float(np.mean([a.elapsed_time(b) for a, b in self.pairs]))


def eager_steps(run, steps, warmup):
    """Warmup, then ``steps`` steps with events around each launch (the
    per-kernel times), then ``steps`` steps without events, timed as a whole
    between two synchronizations: the step time.  Returns seconds per step."""
    for _ in range(warmup):
        run(False)
    torch.cuda.synchronize()
    for _ in range(steps):
        run(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run(False)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


# --------------------------------------------------------------------------
def decode_nf4(dev, steps, warmup, M=1):
    """Qwen3 NF4 decode: gate_up GEMV + down GEMV per step (graph replay)."""
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (Ng, Kg), (Nd, Kd) = wl.QWEN["gate_up"], wl.QWEN["down"]
    banks_g = [wl.random_nf4_bank(E, Ng, Kg, dev, seed=10 + c) for c in range(COPIES)]
    banks_d = [wl.random_nf4_bank(E, Nd, Kd, dev, seed=100 + c) for c in range(COPIES)]
    g = wl.rng(wl.CFG_QWEN_DECODE, wl.S_ROUTE)
    ids = [wl.route_uniform(g, M, E, topk) for _ in range(steps + warmup)]
    ids_g = [torch.from_numpy(i).to(dev) for i in ids]
    ids_d = [torch.from_numpy(i.reshape(-1, 1).copy()).to(dev) for i in ids]
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_X), (M, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_DOWN_IN), (M * topk, Kd)), dev)
    out_g = torch.empty((M * topk, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((M * topk, Nd), dtype=torch.bfloat16, device=dev)

    def gate(i):
        c, a = banks_g[i % COPIES]
        gq.gq_nf4_grouped_gemv(x, c, a, ids_g[i], out=out_g)

    def down(i):
        c, a = banks_d[i % COPIES]
        gq.gq_nf4_grouped_gemv(xd, c, a, ids_d[i], out=out_d)

    def step(i):
        gate(i)
        down(i)

    for i in range(steps, steps + warmup):            # untimed warmup steps (eager)
        step(i)
    g_steps = capture(step, steps)
    g_gate = capture(gate, steps)
    g_steps.replay()                                   # first replay uploads the graph
    g_gate.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gate_ms = event_ms(g_gate.replay)

    def step_bytes(i):
        d = len(set(ids[i].reshape(-1).tolist()))
        bg = d * nf4_expert_bytes(Ng, Kg) + M * Kg * 2 + M * topk * Ng * 2
        bd = d * nf4_expert_bytes(Nd, Kd) + M * topk * Kd * 2 + M * topk * Nd * 2
        return bg, bd

    byts = [step_bytes(i) for i in range(steps)]
    total = sum(a + b for a, b in byts)
    gate_bytes = float(np.mean([a for a, _ in byts]))
    gate_us = 1e3 * gate_ms / steps
    sample = {"ids": ids[:steps], "banks_g": banks_g, "banks_d": banks_d, "x": x, "xd": xd}
    return {
        "ms_per_step": 1e3 * dt / steps,
        "gbs": total / dt / 1e9,
        "bytes_per_step": total / steps,
        "gate_up_bytes_per_launch": gate_bytes,
        "gate_up_us": gate_us,
        "gate_up_gbs": gate_bytes / (gate_us * 1e-6) / 1e9,
    }, sample


def controls(dev, nbytes, n=64):
    """Empty-launch floor and a cold streaming read of nbytes, graph-replayed."""
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_grouped_moe_amd", "libgq_probes.so"))
    lib.gq_probe_empty.argtypes = [ctypes.c_void_p]
    lib.gq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.gq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_void_p]
    nb = (nbytes + 15) // 16 * 16
    nbuf = 40                                          # 40 x 14 MB >> the 256 MB cache
    bufs = [torch.randint(0, 255, (nb,), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def stream(i):
        st = lib.gq_probe_stream_read(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nb,
                                      ctypes.c_void_p(sink.data_ptr()),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0

    def empty(i):
        assert lib.gq_probe_empty(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0

    dst = torch.empty(nb, dtype=torch.uint8, device=dev)

    def copy(i):
        st = lib.gq_probe_copy(ctypes.c_void_p(bufs[i % nbuf].data_ptr()),
                               ctypes.c_void_p(dst.data_ptr()), nb,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0

    gs, ge, gc = capture(stream, n), capture(empty, n), capture(copy, n)
    gs.replay()
    ge.replay()
    gc.replay()
    us_stream = 1e3 * event_ms(gs.replay) / n
    us_empty = 1e3 * event_ms(ge.replay) / n
    us_copy = 1e3 * event_ms(gc.replay) / n
    return {"empty_launch_us": us_empty, "stream_read_us": us_stream,
            "stream_read_gbs": nb / (us_stream * 1e-6) / 1e9, "stream_read_bytes": nb,
            "copy_us": us_copy, "copy_gbs": 2 * nb / (us_copy * 1e-6) / 1e9}


def decode_mx(dev, steps, warmup):
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    (Ng, Kg), (Nd, Kd) = wl.GPTOSS["gate_up"], wl.GPTOSS["down"]
    copies = 8
    banks_g = [wl.random_mxfp4_bank(E, Ng, Kg, dev, seed=20 + c) for c in range(copies)]
    banks_d = [wl.random_mxfp4_bank(E, Nd, Kd, dev, seed=200 + c) for c in range(copies)]
    g = wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE)
    ids = [wl.route_uniform(g, 1, E, topk) for _ in range(steps + warmup)]
    ids_g = [torch.from_numpy(i).to(dev) for i in ids]
    ids_d = [torch.from_numpy(i.reshape(-1, 1).copy()).to(dev) for i in ids]
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X), (1, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_DOWN_IN), (topk, Kd)), dev)
    out_g = torch.empty((topk, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((topk, Nd), dtype=torch.bfloat16, device=dev)

    def gate(i):
        b, s = banks_g[i % copies]
        gq.gq_mxfp4_grouped_gemv(x, b, s, ids_g[i], out=out_g)

    def step(i):
        gate(i)
        b, s = banks_d[i % copies]
        gq.gq_mxfp4_grouped_gemv(xd, b, s, ids_d[i], out=out_d)

    for i in range(steps, steps + warmup):
        step(i)
    g_steps, g_gate = capture(step, steps), capture(gate, steps)
    g_steps.replay()
    g_gate.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    us = 1e3 * event_ms(g_gate.replay) / steps
    bg = topk * mx_expert_bytes(Ng, Kg) + Kg * 2 + topk * Ng * 2
    bd = topk * mx_expert_bytes(Nd, Kd) + topk * Kd * 2 + topk * Nd * 2
    return {"workload": "gpt-oss-20b mxfp4 decode gemv M=1 (gate_up [5760,2880] + down "
                        "[2880,2880], E=32, top-4)",
            "ms_per_step": 1e3 * dt / steps, "gbs": (bg + bd) * steps / dt / 1e9,
            "gate_up_us": us, "gate_up_gbs": bg / (us * 1e-6) / 1e9,
            "gate_up_frac_hbm": bg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}


def decode_layer_nf4(dev, steps, warmup, M=1):
    """Qwen3 NF4 MoE layer, decode: SwiGLU-fused gate_up GEMV + down GEMV with
    the router-weighted combine fused (two launches per step, graph-replayed,
    cold bank copy per step).  Bytes: active experts' packed weights, x, y."""
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (Ng, Kg), (Nd, Kd) = wl.QWEN["gate_up"], wl.QWEN["down"]
    banks_g = [wl.random_nf4_bank(E, Ng, Kg, dev, seed=50 + c) for c in range(COPIES)]
    banks_d = [wl.random_nf4_bank(E, Nd, Kd, dev, seed=500 + c) for c in range(COPIES)]
    g = wl.rng(wl.CFG_QWEN_DECODE, 70)
    ids = [wl.route_uniform(g, M, E, topk) for _ in range(steps + warmup)]
    t_ids = [torch.from_numpy(i).to(dev) for i in ids]
    tw = torch.from_numpy(wl.router_weights(g, M, topk)).to(dev)
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, 71), (M, Kg)), dev)
    act = torch.empty((M * topk, Ng // 2), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, Nd), dtype=torch.bfloat16, device=dev)

    def step(i):
        c, a = banks_g[i % COPIES]
        gq.gq_nf4_grouped_gemv_swiglu(x, c, a, t_ids[i], out=act)
        c, a = banks_d[i % COPIES]
        gq.gq_nf4_grouped_gemv_down_combine(act, c, a, t_ids[i], tw, out=y)

    for i in range(steps, steps + warmup):
        step(i)
    gr = capture(step, steps)
    gr.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gr.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    total = 0
    for i in range(steps):
        d = len(set(ids[i].reshape(-1).tolist()))
        total += d * (nf4_expert_bytes(Ng, Kg) + nf4_expert_bytes(Nd, Kd)) + M * Kg * 2 + M * Nd * 2
    return {"workload": f"qwen3-30b-a3b nf4 moe layer decode M={M}: swiglu gate_up gemv + "
                        f"down gemv with router-weighted combine (2 launches)",
            "ms_per_step": 1e3 * dt / steps, "gbs": total / dt / 1e9,
            "bytes_per_step": total / steps}


def prefill_layer_nf4(dev, steps, warmup):
    """Qwen3 NF4 MoE layer, prefill (M=4096 Zipf top-8): route sort + SwiGLU-
    fused gate_up GEMM + down GEMM (router weight as pair scale) + combine."""
    cfgd, M, cfg = wl.QWEN, 4096, wl.CFG_QWEN_PREFILL
    E, topk = cfgd["E"], cfgd["topk"]
    (Ng, Kg), (Nd, Kd) = cfgd["gate_up"], cfgd["down"]
    P = M * topk
    route = wl.route_zipf(wl.rng(cfg, wl.S_ROUTE), M, E, topk)
    cg, ag = wl.random_nf4_bank(E, Ng, Kg, dev, seed=31)
    cd, ad = wl.random_nf4_bank(E, Nd, Kd, dev, seed=301)
    ids = torch.from_numpy(route).to(dev)
    sc = torch.from_numpy(wl.router_weights(wl.rng(cfg, wl.S_LOGITS), M, topk)).to(dev)
    x = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_X), (M, Kg)), dev)
    act = torch.empty((P, Ng // 2), dtype=torch.bfloat16, device=dev)
    yp = torch.empty((P, Nd), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, Nd), dtype=torch.bfloat16, device=dev)
    tg, td, tc = Timer(), Timer(), Timer()

    def run(timed):
        r = gq.gq_route_sort(ids, E)
        rd = r._replace(rows=P, topk=1)
        ev = tg.start() if timed else None
        gq.gq_nf4_grouped_gemm_swiglu(x, cg, ag, r, out=act)
        if timed:
            tg.stop(ev)
            ev = td.start()
        gq.gq_nf4_grouped_gemm(act, cd, ad, rd, pair_scale=sc, out=yp)
        if timed:
            td.stop(ev)
            ev = tc.start()
        gq.gq_moe_combine(yp, topk, out=y)
        if timed:
            tc.stop(ev)

    dt = eager_steps(run, steps, warmup) * steps
    flops = 2.0 * P * (Ng * Kg + Nd * Kd)
    return {"workload": "qwen3-30b-a3b nf4 moe layer prefill M=4096 top-8 Zipf(1.1): route sort "
                        "+ swiglu gate_up gemm + down gemm (router-weight scale) + combine",
            "ms_per_step": 1e3 * dt / steps, "tflops": flops * steps / dt / 1e12,
            "gate_up_swiglu_us": tg.avg_us(), "down_us": td.avg_us(), "combine_us": tc.avg_us(),
            "combine_gbs": (P * Nd * 2 + M * Nd * 2) / (tc.avg_us() * 1e-6) / 1e9}


def prefill(dev, steps, warmup, fmt):
    """NF4 Qwen3 (M=4096 Zipf top-8) or MXFP4 gpt-oss (M=2048 uniform top-4):
    route sort + gate_up GEMM + down GEMM per step (eager; kernels are long)."""
    if fmt == "nf4":
        cfgd, M, cfg = wl.QWEN, 4096, wl.CFG_QWEN_PREFILL
        route = wl.route_zipf(wl.rng(cfg, wl.S_ROUTE), M, cfgd["E"], cfgd["topk"])
        bank = wl.random_nf4_bank
        fn = gq.gq_nf4_grouped_gemm
    else:
        cfgd, M, cfg = wl.GPTOSS, 2048, wl.CFG_GPTOSS
        route = wl.route_uniform(wl.rng(cfg, wl.S_ROUTE), M, cfgd["E"], cfgd["topk"])
        bank = wl.random_mxfp4_bank
        fn = gq.gq_mxfp4_grouped_gemm
    E, topk = cfgd["E"], cfgd["topk"]
    (Ng, Kg), (Nd, Kd) = cfgd["gate_up"], cfgd["down"]
    P = M * topk
    a_g, b_g = bank(E, Ng, Kg, dev, seed=30)
    a_d, b_d = bank(E, Nd, Kd, dev, seed=300)
    ids = torch.from_numpy(route).to(dev)
    sc = torch.from_numpy(wl.router_weights(wl.rng(cfg, wl.S_LOGITS), M, topk)).to(dev)
    x = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_X), (M, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_DOWN_IN), (P, Kd)), dev)
    out_g = torch.empty((P, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((P, Nd), dtype=torch.bfloat16, device=dev)
    tg, td, ts = Timer(), Timer(), Timer()

    def run(timed):
        ev = ts.start() if timed else None
        r = gq.gq_route_sort(ids, E)
        rd = r._replace(rows=P, topk=1)          # same grouping, flatten mode for down
        if timed:
            ts.stop(ev)
            ev = tg.start()
        fn(x, a_g, b_g, r, pair_scale=sc, out=out_g)
        if timed:
            tg.stop(ev)
            ev = td.start()
        fn(xd, a_d, b_d, rd, pair_scale=sc, out=out_d)
        if timed:
            td.stop(ev)

    dt = eager_steps(run, steps, warmup) * steps
    fg, fd = 2.0 * P * Ng * Kg, 2.0 * P * Nd * Kd
    ug, ud, us = tg.avg_us(), td.avg_us(), ts.avg_us()
    counts = np.bincount(route.reshape(-1), minlength=E)
    eb = nf4_expert_bytes(Ng, Kg) if fmt == "nf4" else mx_expert_bytes(Ng, Kg)
    return {
        "gate_up_bytes": int((counts > 0).sum()) * eb + M * Kg * 2 + P * Ng * 2,
        "ms_per_step": 1e3 * dt / steps,
        "tflops": (fg + fd) * steps / dt / 1e12,
        "gate_up_us": ug, "down_us": ud, "route_sort_us": us,
        "gate_up_tflops": fg / (ug * 1e-6) / 1e12,
        "down_tflops": fd / (ud * 1e-6) / 1e12,
        "expert_rows_max_median_min": [int(counts.max()), float(np.median(counts)),
                                       int(counts.min())],
    }


def dgrad(dev, steps, warmup, fmt="nf4"):
    """Input gradient of both projections: Qwen3 NF4 (M=2048 top-8) or
    gpt-oss MXFP4 (M=2048 top-4), eager."""
    if fmt == "nf4":
        cfgd, cfg, bank, fn = wl.QWEN, wl.CFG_QWEN_DGRAD, wl.random_nf4_bank, gq.gq_nf4_grouped_dgrad
    else:
        cfgd, cfg, bank, fn = wl.GPTOSS, wl.CFG_GPTOSS, wl.random_mxfp4_bank, gq.gq_mxfp4_grouped_dgrad
    E, topk = cfgd["E"], cfgd["topk"]
    (Ng, Kg), (Nd, Kd) = cfgd["gate_up"], cfgd["down"]
    M = 2048
    P = M * topk
    pe = wl.route_uniform(wl.rng(cfg, wl.S_ROUTE), M, E, topk).reshape(-1, 1)
    ids = torch.from_numpy(pe.copy()).to(dev)
    cg, ag = bank(E, Ng, Kg, dev, seed=40)
    cd, ad = bank(E, Nd, Kd, dev, seed=400)
    dyg = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_DOWN_IN), (P, Ng)), dev)
    dyd = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_X), (P, Nd)), dev)
    tg, td = Timer(), Timer()

    def run(timed):
        r = gq.gq_route_sort(ids, E)
        ev = tg.start() if timed else None
        fn(dyg, cg, ag, r)
        if timed:
            tg.stop(ev)
            ev = td.start()
        fn(dyd, cd, ad, r)
        if timed:
            td.stop(ev)

    dt = eager_steps(run, steps, warmup) * steps
    fg, fd = 2.0 * P * Ng * Kg, 2.0 * P * Nd * Kd
    ug, ud = tg.avg_us(), td.avg_us()
    name = ("qwen3-30b-a3b nf4 dgrad M=2048 top-8 (16384 pairs)" if fmt == "nf4" else
            "gpt-oss-20b mxfp4 dgrad M=2048 top-4 (8192 pairs)")
    return {"workload": name,
            "ms_per_step": 1e3 * dt / steps, "tflops": (fg + fd) * steps / dt / 1e12,
            "gate_up_us": ug, "down_us": ud,
            "gate_up_tflops": fg / (ug * 1e-6) / 1e12, "down_tflops": fd / (ud * 1e-6) / 1e12}


# --------------------------------------------------------------------------
def cpu_baseline(sample, budget_s):
    """The oracle as it stands: decode of the active experts + float64
    grouped matmul, for as many decode steps as fit in the time budget
    (at least one).  BLAS is held to one thread, so ``cores`` is exact."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits = None
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (Ng, Kg), (Nd, Kd) = wl.QWEN["gate_up"], wl.QWEN["down"]
    x_bits = sample["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    xd_bits = sample["xd"].view(torch.int16).cpu().numpy().view(np.uint16)
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    done, total_bytes, elapsed = 0, 0, 0.0
    try:
        for i, ids in enumerate(sample["ids"]):
            cg, ag = sample["banks_g"][i % COPIES]
            cd, ad = sample["banks_d"][i % COPIES]
            active = sorted(set(ids.reshape(-1).tolist()))
            host = {e: (cg[e].cpu().numpy(), ag[e].cpu().numpy(), cd[e].cpu().numpy(),
                        ad[e].cpu().numpy()) for e in active}          # untimed host copy
            t0 = time.perf_counter()
            wg = {e: oracle.nf4_decode(host[e][0], host[e][1]) for e in active}
            wd = {e: oracle.nf4_decode(host[e][2], host[e][3]) for e in active}
            oracle.grouped_gemm(x_bits, lambda e: wg[e], ids, E)
            oracle.grouped_gemm(xd_bits, lambda e: wd[e], ids.reshape(-1, 1), E)
            elapsed += time.perf_counter() - t0
            done += 1
            d = len(active)
            total_bytes += (d * (nf4_expert_bytes(Ng, Kg) + nf4_expert_bytes(Nd, Kd))
                            + Kg * 2 + topk * Ng * 2 + topk * Kd * 2 + topk * Nd * 2)
            if elapsed >= budget_s:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return {"value": total_bytes / elapsed / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of the timed decode steps (M=1, gate_up + down, 8 experts each): "
                      f"NumPy NF4 decode of the active experts + float64 grouped matmul, "
                      f"{elapsed:.1f} s on 1 core (BLAS limited to 1 thread)"}


def measured_traffic(kernel_key, algorithmic):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    from bit_grouped_moe_amd.profile_summary import sources_sha
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if sources_sha(kernel_key) != rec["source_sha256"]:
        return None
    return {"bytes_per_launch": round(rec["hbm_bytes_per_launch"]),
            "read_bytes": round(rec["fetch_bytes"]), "written_bytes": round(rec["write_bytes"]),
            "ratio_to_algorithmic": round(rec["hbm_bytes_per_launch"] / algorithmic, 4)}


def traffic_bytes(t):
    return None if t is None else t["bytes_per_launch"]


def r4(d):
    return {k: (round(v, 4) if isinstance(v, float) else v) for k, v in d.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--prefill-steps", type=int, default=30)
    ap.add_argument("--prefill-warmup", type=int, default=30,
                    help="untimed prefill/dgrad steps first (long kernels: lets the clocks settle)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--quick", action="store_true", help="headline + prefill only, short CPU leg")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(expert-parallel sharding is a design note only); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    gq.load_library()
    dev = torch.device("cuda:0")

    log("[bench] nf4 decode M=1")
    dec, sample = decode_nf4(dev, args.steps, args.warmup, M=1)
    log("[bench]", r4(dec))
    ctl = controls(dev, int(dec["gate_up_bytes_per_launch"]))
    log("[bench] controls", r4(ctl))
    log("[bench] nf4 prefill M=4096")
    pre = prefill(dev, args.prefill_steps, args.prefill_warmup, "nf4")
    log("[bench]", r4(pre))
    extra = {}
    if not args.quick:
        log("[bench] nf4 decode M=4")
        d4, _ = decode_nf4(dev, args.steps, args.warmup, M=4)
        extra["nf4_decode_m4"] = {"workload": "qwen3-30b-a3b nf4 decode gemv M=4", **d4,
                                  "gate_up_frac_hbm": d4["gate_up_gbs"] / HBM_PEAK_GBS}
        log("[bench] mxfp4 decode M=1")
        extra["mxfp4_decode_m1"] = decode_mx(dev, args.steps, args.warmup)
        log("[bench] mxfp4 prefill M=2048")
        mp = prefill(dev, args.prefill_steps, args.prefill_warmup, "mx")
        mp["workload"] = "gpt-oss-20b mxfp4 prefill M=2048 top-4 (bf16 MFMA on exact decode)"
        mp["gate_up_frac_bf16_peak"] = mp["gate_up_tflops"] / BF16_PEAK_TFLOPS
        mp["gate_up_frac_fp4_peak"] = mp["gate_up_tflops"] / FP4_PEAK_TFLOPS
        extra["mxfp4_prefill_m2048"] = mp
        log("[bench] nf4 moe layer decode M=1")
        extra["nf4_moe_layer_decode_m1"] = decode_layer_nf4(dev, args.steps, args.warmup)
        log("[bench] nf4 moe layer prefill M=4096")
        extra["nf4_moe_layer_prefill_m4096"] = prefill_layer_nf4(dev, args.prefill_steps,
                                                                 args.prefill_warmup)
        log("[bench] nf4 dgrad")
        extra["nf4_dgrad_m2048"] = dgrad(dev, args.prefill_steps, args.prefill_warmup)
        log("[bench] mxfp4 dgrad")
        extra["mxfp4_dgrad_m2048"] = dgrad(dev, args.prefill_steps, args.prefill_warmup, "mx")
    extra = {k: r4(v) for k, v in extra.items()}

    log("[bench] cpu baseline (oracle)")
    cpu = cpu_baseline(sample, 3.0 if args.quick else args.cpu_budget)

    gemv_traffic = measured_traffic("gemv_nf4_gate_up_m1", dec["gate_up_bytes_per_launch"])
    gemm_traffic = measured_traffic("gemm_nf4_gate_up_prefill", pre["gate_up_bytes"])
    line = {
        "metric": "decode GB/s (% HBM peak) @1 tok; prefill TFLOP/s (% MFMA peak) @4096 tok",
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwen3-30b-a3b-shaped nf4 decode gemv, M=1 token, top-8 of "
                               "E=128, gate_up W[1536,2048] + down W[2048,768], own routing "
                               "and cold bank copy per step, graph-replayed",
                   "bytes_per_step": round(dec["bytes_per_step"]),
                   "frac_hbm_peak": round(dec["gbs"] / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(dec["gate_up_gbs"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec["gate_up_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic_bytes(gemv_traffic),
                     "traffic_detail": gemv_traffic,
                     "kernel": "grouped_gemv_kernel (NF4, gate_up, M=1)",
                     "bytes_per_launch": round(dec["gate_up_bytes_per_launch"]),
                     "avg_launch_us": round(dec["gate_up_us"], 3),
                     "controls": r4(ctl)},
        "cpu_baseline": r4(cpu),
        "prefill": {"workload": "qwen3-30b-a3b-shaped nf4 prefill, M=4096 tokens, top-8 Zipf(1.1) "
                                "of E=128, router-weight scales: route sort + gate_up GEMM + "
                                "down GEMM",
                    "value": round(pre["tflops"], 2), "unit": "TFLOP/s", "dtype": "bf16",
                    "ms_per_step": round(pre["ms_per_step"], 4),
                    "roofline": {"bound": "mfma", "achieved": round(pre["gate_up_tflops"], 2),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(pre["gate_up_tflops"] / BF16_PEAK_TFLOPS, 4),
                                 "traffic": traffic_bytes(gemm_traffic),
                                 "traffic_detail": gemm_traffic,
                                 "kernel": "grouped_gemm_fwd_kernel (NF4, gate_up)",
                                 "avg_launch_us": round(pre["gate_up_us"], 2)},
                    "down_tflops": round(pre["down_tflops"], 2),
                    "down_us": round(pre["down_us"], 2),
                    "route_sort_us": round(pre["route_sort_us"], 2),
                    "expert_rows_max_median_min": pre["expert_rows_max_median_min"]},
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
