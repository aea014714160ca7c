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
    graph of max(K, 200) gate_up launches on the launch stream (a short K
    would charge the graph's own launch overhead to the kernel), against
    the 8 TB/s HBM peak; plus same-run controls: the empty-launch floor and a plain
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
FP8_PEAK_TFLOPS = 5033.0         # MI355X dense fp8 MFMA
FP4_PEAK_TFLOPS = 10066.0        # MI355X dense fp4 MFMA
COPIES = 16                      # independent bank copies rotated per step
# Per-kernel decode timings (the roofline and the additive fit) replay a graph
# of at least this many launches of the one kernel, so that the graph's own
# launch overhead is not charged to the kernel when --steps is small (at K =
# 20 it added ~0.5 us to each one-token GEMV); the headline's timed region is
# still exactly K steps.
KERNEL_LAUNCHES = 200
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
    # the down product reads the same routing tensor, flattened (a view), as
    # in a real layer where both projections consume one router output
    ids_d = [t.view(-1, 1) for t in ids_g]
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_X), (M, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_DOWN_IN), (M * topk, Kd)), dev)
    out_g = torch.empty((M * topk, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((M * topk, Nd), dtype=torch.bfloat16, device=dev)

    n_ids = len(ids_g)

    def gate(i):
        c, a = banks_g[i % COPIES]
        gq.gq_nf4_grouped_gemv(x, c, a, ids_g[i % n_ids], out=out_g)

    def down(i):
        c, a = banks_d[i % COPIES]
        gq.gq_nf4_grouped_gemv(xd, c, a, ids_d[i % n_ids], out=out_d)

    def step(i):
        gate(i)
        down(i)

    for i in range(steps, steps + warmup):            # untimed warmup steps (eager)
        step(i)
    nk = max(steps, KERNEL_LAUNCHES)
    g_steps = capture(step, steps)
    g_gate = capture(gate, nk)
    g_down = capture(down, nk)
    g_steps.replay()                                   # first replay uploads the graph
    g_gate.replay()
    g_down.replay()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gate_ms = event_ms(g_gate.replay)
    down_ms = event_ms(g_down.replay)

    def step_bytes(i):
        d = len(set(ids[i].reshape(-1).tolist()))
        bg = d * nf4_expert_bytes(Ng, Kg) + M * Kg * 2 + M * topk * Ng * 2
        bd = d * nf4_expert_bytes(Nd, Kd) + M * topk * Kd * 2 + M * topk * Nd * 2
        return bg, bd

    total = sum(a + b for a, b in (step_bytes(i) for i in range(steps)))
    kbyts = [step_bytes(i % n_ids) for i in range(nk)]     # the kernel graphs' launches
    gate_bytes = float(np.mean([a for a, _ in kbyts]))
    down_bytes = float(np.mean([b for _, b in kbyts]))
    gate_us = 1e3 * gate_ms / nk
    down_us = 1e3 * down_ms / nk
    sample = {"ids": ids[:steps], "banks_g": banks_g, "banks_d": banks_d, "x": x, "xd": xd}
    return {
        "ms_per_step": 1e3 * dt / steps,
        "gbs": total / dt / 1e9,
        "bytes_per_step": total / steps,
        "gate_up_bytes_per_launch": gate_bytes,
        "gate_up_us": gate_us,
        "gate_up_gbs": gate_bytes / (gate_us * 1e-6) / 1e9,
        "down_bytes_per_launch": down_bytes,
        "down_us": down_us,
        "down_gbs": down_bytes / (down_us * 1e-6) / 1e9,
    }, sample


def probes_lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "bit_grouped_moe_amd", "libgq_probes.so"))
    lib.gq_probe_empty.argtypes = [ctypes.c_void_p]
    lib.gq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.gq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_void_p]
    lib.gq_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.gq_probe_mfma_flops.argtypes = [ctypes.c_int32]
    lib.gq_probe_mfma_flops.restype = ctypes.c_int64
    lib.gq_probe_mfma_per_wave_iter.restype = ctypes.c_int32
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def fit_line(xs, ys):
    """Least-squares t = t0 + bytes / bw over the points (bytes, us):
    returns (t0_us, bw_gbs)."""
    A = np.stack([np.ones(len(xs)), np.asarray(xs, dtype=np.float64)], axis=1)
    (t0, slope), *_ = np.linalg.lstsq(A, np.asarray(ys, dtype=np.float64), rcond=None)
    return float(t0), float(1e-3 / slope) if slope > 0 else float("inf")


def controls(dev, sizes, n=64):
    """Same-run controls, graph-replayed: the empty-launch floor, a plain copy
    of sizes[0] bytes, and a cold streaming read of every size in ``sizes``
    (each at 1, 4 and 16 loads per thread; the fastest shape is the control
    for that size), plus the fit t = t0 + bytes/bw over the stream sizes."""
    lib = probes_lib()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    out = {"stream": []}
    for nbytes in sizes:
        nb = (int(nbytes) + 15) // 16 * 16
        nbuf = max(4, -(-600_000_000 // nb))           # > 2x the 256 MB last-level cache
        bufs = [torch.randint(0, 255, (nb,), dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        best = None
        for L in (1, 4, 16):
            def stream(i, L=L):
                assert lib.gq_probe_stream_read(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nb, L,
                                                ctypes.c_void_p(sink.data_ptr()), _stream()) == 0
            gs = capture(stream, n)
            gs.replay()
            us = 1e3 * event_ms(gs.replay) / n
            if best is None or us < best[1]:
                best = (L, us)
        out["stream"].append({"bytes": nb, "us": best[1], "gbs": nb / (best[1] * 1e-6) / 1e9,
                              "loads_per_thread": best[0]})
        if nbytes == sizes[0]:
            dst = torch.empty(nb, dtype=torch.uint8, device=dev)

            def copy(i):
                assert lib.gq_probe_copy(ctypes.c_void_p(bufs[i % nbuf].data_ptr()),
                                         ctypes.c_void_p(dst.data_ptr()), nb, _stream()) == 0
            gc = capture(copy, n)
            gc.replay()
            us_copy = 1e3 * event_ms(gc.replay) / n
            out["copy_us"] = us_copy
            out["copy_gbs"] = 2 * nb / (us_copy * 1e-6) / 1e9
            del dst
        del bufs

    def empty(i):
        assert lib.gq_probe_empty(_stream()) == 0

    ge = capture(empty, n)
    ge.replay()
    out["empty_launch_us"] = 1e3 * event_ms(ge.replay) / n
    t0, bw = fit_line([s["bytes"] for s in out["stream"]], [s["us"] for s in out["stream"]])
    out["stream_fit"] = {"t0_us": t0, "bw_gbs": bw, "bw_frac_hbm": bw / HBM_PEAK_GBS}
    return out


def mfma_rates(dev, iters=4096, blocks=1024, launches=12):
    """Dense matrix-instruction rates on this GPU (random operands, four
    waves per SIMD): bf16 32x32x16 and the block-scaled 32x32x64 f8f6f4
    instruction with e4m3 x e2m1, e2m1 x e2m1 and e4m3 x e4m3 operands.
    Each kind runs ``launches`` launches back to back; the rate is taken
    over the last half (the clock settles under sustained load)."""
    lib = probes_lib()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    per_iter = lib.gq_probe_mfma_per_wave_iter()
    names = {0: "bf16_32x32x16", 1: "scale_e4m3_x_e2m1_32x32x64",
             2: "scale_e2m1_x_e2m1_32x32x64", 3: "scale_e4m3_x_e4m3_32x32x64"}
    res = {}
    for kind, name in names.items():
        flops = lib.gq_probe_mfma_flops(kind) * per_iter * iters * blocks * 4
        times = []
        for _ in range(launches):
            times.append(event_ms(lambda: lib.gq_probe_mfma(kind, iters, blocks,
                                                             ctypes.c_void_p(sink.data_ptr()),
                                                             _stream())))
        ms = float(np.median(times[launches // 2:]))
        insts = per_iter * iters * blocks * 4
        res[name] = {"tflops": flops / (ms * 1e-3) / 1e12,
                     "ns_per_inst_per_simd": ms * 1e6 / (insts / 1024)}
    bf = res["bf16_32x32x16"]["tflops"]
    for name in names.values():
        res[name]["vs_bf16_flop_rate"] = res[name]["tflops"] / bf
    return res


def decode_mx(dev, steps, warmup):
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    (Ng, Kg), (Nd, Kd) = wl.GPTOSS["gate_up"], wl.GPTOSS["down"]
    copies = 8
    banks_g = [wl.random_mxfp4_bank(E, Ng, Kg, dev, seed=20 + c) for c in range(copies)]
    banks_d = [wl.random_mxfp4_bank(E, Nd, Kd, dev, seed=200 + c) for c in range(copies)]
    g = wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE)
    ids = [wl.route_uniform(g, 1, E, topk) for _ in range(steps + warmup)]
    ids_g = [torch.from_numpy(i).to(dev) for i in ids]
    # the down product reads the same routing tensor, flattened (a view), as
    # in a real layer where both projections consume one router output
    ids_d = [t.view(-1, 1) for t in ids_g]
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X), (1, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_DOWN_IN), (topk, Kd)), dev)
    out_g = torch.empty((topk, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((topk, Nd), dtype=torch.bfloat16, device=dev)

    n_ids = len(ids_g)

    def gate(i):
        b, s = banks_g[i % copies]
        gq.gq_mxfp4_grouped_gemv(x, b, s, ids_g[i % n_ids], out=out_g)

    def down(i):
        b, s = banks_d[i % copies]
        gq.gq_mxfp4_grouped_gemv(xd, b, s, ids_d[i % n_ids], out=out_d)

    def step(i):
        gate(i)
        down(i)

    for i in range(steps, steps + warmup):
        step(i)
    nk = max(steps, KERNEL_LAUNCHES)
    g_steps, g_gate, g_down = capture(step, steps), capture(gate, nk), capture(down, nk)
    g_steps.replay()
    g_gate.replay()
    g_down.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    us = 1e3 * event_ms(g_gate.replay) / nk
    us_d = 1e3 * event_ms(g_down.replay) / nk
    bg = topk * mx_expert_bytes(Ng, Kg) + Kg * 2 + topk * Ng * 2
    bd = topk * mx_expert_bytes(Nd, Kd) + topk * Kd * 2 + topk * Nd * 2
    return {"workload": "gpt-oss-20b mxfp4 decode gemv M=1 (gate_up [5760,2880] + down "
                        "[2880,2880], E=32, top-4)",
            "ms_per_step": 1e3 * dt / steps, "gbs": (bg + bd) * steps / dt / 1e9,
            "gate_up_bytes_per_launch": bg, "down_bytes_per_launch": bd,
            "gate_up_us": us, "gate_up_gbs": bg / (us * 1e-6) / 1e9,
            "gate_up_frac_hbm": bg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "down_us": us_d, "down_gbs": bd / (us_d * 1e-6) / 1e9}


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


def decode_layer_mx(dev, steps, warmup, M=1):
    """gpt-oss-20b MXFP4 MoE layer, decode: gate_up GEMV with the gpt-oss
    gated unit + down GEMV with the router-weighted combine fused (two
    launches per step, graph-replayed, cold bank copy per step)."""
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    (Ng, Kg), (Nd, Kd) = wl.GPTOSS["gate_up"], wl.GPTOSS["down"]
    copies = 8                                     # 8 x 332 MB of banks > the last-level cache
    banks_g = [wl.random_mxfp4_bank(E, Ng, Kg, dev, seed=60 + c) for c in range(copies)]
    banks_d = [wl.random_mxfp4_bank(E, Nd, Kd, dev, seed=600 + c) for c in range(copies)]
    g = wl.rng(wl.CFG_GPTOSS, 72)
    ids = [wl.route_uniform(g, M, E, topk) for _ in range(steps + warmup)]
    t_ids = [torch.from_numpy(i).to(dev) for i in ids]
    tw = torch.from_numpy(wl.router_weights(g, M, topk)).to(dev)
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, 73), (M, Kg)), dev)
    act = torch.empty((M * topk, Ng // 2), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, Nd), dtype=torch.bfloat16, device=dev)

    def step(i):
        b, s_ = banks_g[i % copies]
        gq.gq_mxfp4_grouped_gemv_swiglu(x, b, s_, t_ids[i], out=act)
        b, s_ = banks_d[i % copies]
        gq.gq_mxfp4_grouped_gemv_down_combine(act, b, s_, t_ids[i], tw, out=y)

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
        total += d * (mx_expert_bytes(Ng, Kg) + mx_expert_bytes(Nd, Kd)) + M * Kg * 2 + M * Nd * 2
    return {"workload": f"gpt-oss-20b mxfp4 moe layer decode M={M}: gate_up gemv with the "
                        f"gpt-oss gated unit + down gemv with router-weighted combine (2 launches)",
            "ms_per_step": 1e3 * dt / steps, "gbs": total / dt / 1e9,
            "bytes_per_step": total / steps, "frac_hbm": total / dt / 1e9 / HBM_PEAK_GBS}


def prefill_layer_mx(dev, steps, warmup):
    """gpt-oss-20b MXFP4 MoE layer, prefill (M=2048 uniform top-4) on the
    block-scaled fp4 instruction: route sort + split + gate_up GEMM with the
    gated unit written as its split + down GEMM (router weight as pair
    scale) + combine."""
    cfgd, M, cfg = wl.GPTOSS, 2048, wl.CFG_GPTOSS
    E, topk = cfgd["E"], cfgd["topk"]
    (Ng, Kg), (Nd, Kd) = cfgd["gate_up"], cfgd["down"]
    P = M * topk
    route = wl.route_uniform(wl.rng(cfg, wl.S_ROUTE), M, E, topk)
    a_g, b_g = wl.random_mxfp4_bank(E, Ng, Kg, dev, seed=32)
    a_d, b_d = wl.random_mxfp4_bank(E, Nd, Kd, dev, seed=302)
    ids = torch.from_numpy(route).to(dev)
    sc = torch.from_numpy(wl.router_weights(wl.rng(cfg, wl.S_LOGITS), M, topk)).to(dev)
    x = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_X), (M, Kg)), dev)
    yp = torch.empty((P, Nd), dtype=torch.bfloat16, device=dev)
    y = torch.empty((M, Nd), dtype=torch.bfloat16, device=dev)
    cs, ss = gq.split_sizes(M, Kg)
    sx = (torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=torch.uint8, device=dev))
    cs, ss = gq.split_sizes(P, Kd)
    sa = (torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=torch.uint8, device=dev))
    tg, td, tc = Timer(), Timer(), Timer()

    def run(timed):
        r = gq.gq_route_sort(ids, E)
        rd = r._replace(rows=P, topk=1)
        gq.gq_act_split_e4m3(x, *sx)
        ev = tg.start() if timed else None
        gq.gq_mxfp4_grouped_gemm_scaled_swiglu_split(sx, a_g, b_g, r, out=sa)
        if timed:
            tg.stop(ev)
        ev = td.start() if timed else None
        gq.gq_mxfp4_grouped_gemm_scaled(sa, a_d, b_d, rd, pair_scale=sc, out=yp)
        if timed:
            td.stop(ev)
            ev = tc.start()
        gq.gq_moe_combine(yp, topk, out=y)
        if timed:
            tc.stop(ev)

    dt = eager_steps(run, steps, warmup) * steps
    flops = 2.0 * P * (Ng * Kg + Nd * Kd)
    return {"workload": "gpt-oss-20b mxfp4 moe layer prefill M=2048 top-4 on the block-scaled "
                        "fp4 instruction: route sort + split + gate_up gemm with the gated unit "
                        "written as its split + down gemm (router-weight scale) + combine",
            "ms_per_step": 1e3 * dt / steps, "tflops": flops * steps / dt / 1e12,
            "gate_up_act_split_us": tg.avg_us(), "down_us": td.avg_us(),
            "combine_us": tc.avg_us()}


def host_stream(dev, steps, warmup, M=1):
    """Qwen3 NF4 decode (M=1, top-8 of 128) with both expert banks in pinned
    host memory: the GEMVs read the routed experts' bytes over the host link
    (graph-replayed, new routing every step).  Controls on the same link:
    a pinned -> device copy of the same byte count (the link ceiling), and
    the copy-then-compute path (the routed experts copied to a device
    staging bank, then the device GEMVs; eager, routing known on the host)."""
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (Ng, Kg), (Nd, Kd) = wl.QWEN["gate_up"], wl.QWEN["down"]
    cg, ag = (t.cpu().pin_memory() for t in wl.random_nf4_bank(E, Ng, Kg, dev, seed=80))
    cd, ad = (t.cpu().pin_memory() for t in wl.random_nf4_bank(E, Nd, Kd, dev, seed=81))
    torch.cuda.synchronize()
    g = wl.rng(wl.CFG_QWEN_DECODE, 82)
    ids = [wl.route_uniform(g, M, E, topk) for _ in range(steps + warmup)]
    ids_g = [torch.from_numpy(i).to(dev) for i in ids]
    # the down product reads the same routing tensor, flattened (a view), as
    # in a real layer where both projections consume one router output
    ids_d = [t.view(-1, 1) for t in ids_g]
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, 83), (M, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, 84), (M * topk, Kd)), dev)
    out_g = torch.empty((M * topk, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((M * topk, Nd), dtype=torch.bfloat16, device=dev)

    def step(i):
        gq.gq_nf4_grouped_gemv_host(x, cg, ag, ids_g[i], out=out_g)
        gq.gq_nf4_grouped_gemv_host(xd, cd, ad, ids_d[i], out=out_d)

    for i in range(steps, steps + warmup):
        step(i)
    gr = capture(step, steps)
    gr.replay()
    torch.cuda.synchronize()
    ms = event_ms(gr.replay) / steps
    d = [len(set(i.reshape(-1).tolist())) for i in ids[:steps]]
    step_bytes = float(np.mean([n * (nf4_expert_bytes(Ng, Kg) + nf4_expert_bytes(Nd, Kd))
                                for n in d])) + M * Kg * 2 + M * topk * (Kd + Ng + Nd) * 2
    # link ceiling: pinned -> device copies of the same byte count, and of 256 MB
    link = {}
    for nb in (int(step_bytes), 256 << 20):
        src = torch.empty(nb, dtype=torch.uint8, pin_memory=True)
        src.fill_(1)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst.copy_(src, non_blocking=True)
        reps = 20 if nb < (64 << 20) else 4
        t = event_ms(lambda: [dst.copy_(src, non_blocking=True) for _ in range(reps)]) / reps
        link[nb] = nb / (t * 1e-3) / 1e9
        del src, dst
    # copy-then-compute: the routed experts to a device staging bank, then the
    # device GEMVs on it (ids remapped to staging slots)
    sg = (torch.empty((topk * M,) + tuple(cg.shape[1:]), dtype=cg.dtype, device=dev),
          torch.empty((topk * M,) + tuple(ag.shape[1:]), dtype=ag.dtype, device=dev))
    sd = (torch.empty((topk * M,) + tuple(cd.shape[1:]), dtype=cd.dtype, device=dev),
          torch.empty((topk * M,) + tuple(ad.shape[1:]), dtype=ad.dtype, device=dev))
    slot_ids = []
    for i in range(steps):
        experts = sorted(set(ids[i].reshape(-1).tolist()))
        remap = {e: j for j, e in enumerate(experts)}
        sid = np.vectorize(remap.get)(ids[i]).astype(np.int32)
        slot_ids.append((experts, torch.from_numpy(sid).to(dev),
                         torch.from_numpy(sid.reshape(-1, 1).copy()).to(dev)))

    def copy_compute(i):
        experts, sid_g, sid_d = slot_ids[i]
        for j, e in enumerate(experts):
            sg[0][j].copy_(cg[e], non_blocking=True)
            sg[1][j].copy_(ag[e], non_blocking=True)
            sd[0][j].copy_(cd[e], non_blocking=True)
            sd[1][j].copy_(ad[e], non_blocking=True)
        gq.gq_nf4_grouped_gemv(x, sg[0][:len(experts)], sg[1][:len(experts)], sid_g, out=out_g)
        gq.gq_nf4_grouped_gemv(xd, sd[0][:len(experts)], sd[1][:len(experts)], sid_d, out=out_d)

    copy_compute(0)
    torch.cuda.synchronize()
    cc_ms = event_ms(lambda: [copy_compute(i) for i in range(steps)]) / steps
    gbs = step_bytes / (ms * 1e-3) / 1e9
    return {"workload": f"qwen3-30b-a3b nf4 decode M={M} (gate_up + down gemv) with both expert "
                        f"banks in pinned host memory, streamed over the host link by the kernel",
            "ms_per_step": ms, "bytes_per_step": step_bytes, "gbs": gbs,
            "link_gbs_same_bytes": link[int(step_bytes)], "link_gbs_256mb": link[256 << 20],
            "frac_of_link": gbs / link[int(step_bytes)],
            "copy_then_compute_ms_per_step": cc_ms,
            "copy_then_compute_gbs": step_bytes / (cc_ms * 1e-3) / 1e9}


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


def dequant_baseline(dev, steps, warmup):
    """The pages' comparator, dequantize-then-GEMM (bit_grouped_moe_amd.dequant_baseline):
    the Qwen3 NF4 decode step (M=1: gate_up + down, own routing, cold bank
    copy per step, graph-replayed) and the Qwen3 NF4 prefill step (M=4096
    Zipf top-8: gate_up + down, one captured step replayed), each the same
    workload as the fused legs; the routing is grouped on the host outside
    the timed region."""
    from bit_grouped_moe_amd.dequant_baseline import DequantGemm
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (Ng, Kg), (Nd, Kd) = wl.QWEN["gate_up"], wl.QWEN["down"]
    res = {}
    # ---- decode M=1 (same banks, routing and inputs as decode_nf4) ----
    banks_g = [wl.random_nf4_bank(E, Ng, Kg, dev, seed=10 + c) for c in range(COPIES)]
    banks_d = [wl.random_nf4_bank(E, Nd, Kd, dev, seed=100 + c) for c in range(COPIES)]
    g = wl.rng(wl.CFG_QWEN_DECODE, wl.S_ROUTE)
    ids = [wl.route_uniform(g, 1, E, topk) for _ in range(steps + warmup)]
    x = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_X), (1, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_DOWN_IN), (topk, Kd)), dev)
    wg = torch.empty((topk, Ng, Kg), dtype=torch.bfloat16, device=dev)
    wd = torch.empty((topk, Nd, Kd), dtype=torch.bfloat16, device=dev)
    dg = [DequantGemm(c, a, wbuf=wg) for c, a in banks_g]
    dd = [DequantGemm(c, a, wbuf=wd) for c, a in banks_d]
    plans = [(dg[0].plan(i, gather=True), dd[0].plan(i.reshape(-1, 1), gather=False))
             for i in ids]
    out_g = torch.empty((topk, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((topk, Nd), dtype=torch.bfloat16, device=dev)

    def step(i):
        pg, pd = plans[i]
        dg[i % COPIES].run(x, pg, out_g)
        dd[i % COPIES].run(xd, pd, out_d)

    for i in range(steps, steps + warmup):
        step(i)
    gr = capture(step, steps)
    gr.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gr.replay()
    torch.cuda.synchronize()
    res["decode_m1_ms_per_step"] = 1e3 * (time.perf_counter() - t0) / steps
    del gr, banks_g, banks_d, dg, dd, wg, wd
    torch.cuda.empty_cache()
    # ---- prefill M=4096 Zipf (same banks, routing and inputs as prefill("nf4")) ----
    cfg, M = wl.CFG_QWEN_PREFILL, 4096
    P = M * topk
    route = wl.route_zipf(wl.rng(cfg, wl.S_ROUTE), M, E, topk)
    cg, ag = wl.random_nf4_bank(E, Ng, Kg, dev, seed=30)
    cd, ad = wl.random_nf4_bank(E, Nd, Kd, dev, seed=300)
    x = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_X), (M, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_DOWN_IN), (P, Kd)), dev)
    pg_ = DequantGemm(cg, ag)
    pd_ = DequantGemm(cd, ad)
    plan_g = pg_.plan(route, gather=True)
    plan_d = pd_.plan(route.reshape(-1, 1), gather=False)
    out_g = torch.empty((P, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((P, Nd), dtype=torch.bfloat16, device=dev)

    def pstep(_):
        pg_.run(x, plan_g, out_g)
        pd_.run(xd, plan_d, out_d)

    def dec_only(_):
        pg_.decode(plan_g)
        pd_.decode(plan_d)

    for _ in range(3):
        pstep(0)
    reps = max(3, min(steps, 10))
    gp = capture(pstep, 1)
    gd = capture(dec_only, 1)
    gp.replay()
    gd.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        gp.replay()
    torch.cuda.synchronize()
    res["prefill_m4096_ms_per_step"] = 1e3 * (time.perf_counter() - t0) / reps
    res["prefill_m4096_dequant_ms"] = event_ms(gd.replay)
    res["prefill_m4096_bf16_copy_bytes"] = E * (Ng * Kg + Nd * Kd) * 2
    return res


def prefill_mx_scaled(dev, steps, warmup):
    """gpt-oss MXFP4 prefill (M=2048 uniform top-4) on the block-scaled fp4
    matrix instruction: route sort + activation split + gate_up GEMM +
    split of the down input + down GEMM per step (eager)."""
    cfgd, M, cfg = wl.GPTOSS, 2048, wl.CFG_GPTOSS
    E, topk = cfgd["E"], cfgd["topk"]
    (Ng, Kg), (Nd, Kd) = cfgd["gate_up"], cfgd["down"]
    P = M * topk
    route = wl.route_uniform(wl.rng(cfg, wl.S_ROUTE), M, E, topk)
    a_g, b_g = wl.random_mxfp4_bank(E, Ng, Kg, dev, seed=30)
    a_d, b_d = wl.random_mxfp4_bank(E, Nd, Kd, dev, seed=300)
    ids = torch.from_numpy(route).to(dev)
    sc = torch.from_numpy(wl.router_weights(wl.rng(cfg, wl.S_LOGITS), M, topk)).to(dev)
    x = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_X), (M, Kg)), dev)
    xd = bf16_dev(wl.draw_bf16(wl.rng(cfg, wl.S_DOWN_IN), (P, Kd)), dev)
    out_g = torch.empty((P, Ng), dtype=torch.bfloat16, device=dev)
    out_d = torch.empty((P, Nd), dtype=torch.bfloat16, device=dev)
    cs, ss = gq.split_sizes(M, Kg)
    sx = (torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=torch.uint8, device=dev))
    cs, ss = gq.split_sizes(P, Kd)
    sxd = (torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=torch.uint8, device=dev))
    t_sg, t_g, t_sd, t_d = Timer(), Timer(), Timer(), Timer()

    def run(timed):
        r = gq.gq_route_sort(ids, E)
        rd = r._replace(rows=P, topk=1)
        ev = t_sg.start() if timed else None
        gq.gq_act_split_e4m3(x, *sx)
        if timed:
            t_sg.stop(ev)
            ev = t_g.start()
        gq.gq_mxfp4_grouped_gemm_scaled(sx, a_g, b_g, r, pair_scale=sc, out=out_g)
        if timed:
            t_g.stop(ev)
            ev = t_sd.start()
        gq.gq_act_split_e4m3(xd, *sxd)
        if timed:
            t_sd.stop(ev)
            ev = t_d.start()
        gq.gq_mxfp4_grouped_gemm_scaled(sxd, a_d, b_d, rd, pair_scale=sc, out=out_d)
        if timed:
            t_d.stop(ev)

    dt = eager_steps(run, steps, warmup) * steps
    fg, fd = 2.0 * P * Ng * Kg, 2.0 * P * Nd * Kd
    ug, ud = t_g.avg_us(), t_d.avg_us()
    return {"workload": "gpt-oss-20b mxfp4 prefill M=2048 top-4 on the block-scaled fp4 matrix "
                        "instruction (e2m1 weights as stored x two-term e4m3 split of the "
                        "activations): route sort + split + gate_up + split + down",
            "ms_per_step": 1e3 * dt / steps, "tflops": (fg + fd) * steps / dt / 1e12,
            "gate_up_us": ug, "down_us": ud, "split_gate_up_us": t_sg.avg_us(),
            "split_down_us": t_sd.avg_us(),
            "gate_up_tflops": fg / (ug * 1e-6) / 1e12, "down_tflops": fd / (ud * 1e-6) / 1e12,
            "gate_up_frac_bf16_peak": fg / (ug * 1e-6) / 1e12 / BF16_PEAK_TFLOPS,
            # two e4m3 x e2m1 instructions per useful product: issued flops are twice the
            # useful ones, against the fp8 x fp4 (fp8-rate) peak
            "gate_up_issued_frac_fp8_peak": 2 * fg / (ug * 1e-6) / 1e12 / FP8_PEAK_TFLOPS,
            "gate_up_frac_fp4_peak": fg / (ug * 1e-6) / 1e12 / FP4_PEAK_TFLOPS}


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
def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def cpu_baseline(sample, budget_s, runs=3):
    """The oracle as it stands: decode of the active experts + float64
    grouped matmul over the timed decode steps, ``runs`` runs of about
    budget_s / runs seconds each; the rate is the median over the runs.
    BLAS gets every core this process may run on (capped by OMP_NUM_THREADS
    where that is set: the host's CPU share); the oracle's decode itself is
    NumPy element-wise work on one thread."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (Ng, Kg), (Nd, Kd) = wl.QWEN["gate_up"], wl.QWEN["down"]
    x_bits = sample["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    xd_bits = sample["xd"].view(torch.int16).cpu().numpy().view(np.uint16)
    affinity = len(os.sched_getaffinity(0))
    share = int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity)
    threads = max(1, min(affinity, share))
    host = {}                                # host copies of active experts (untimed)

    def fetch(i, e):
        key = (i % COPIES, e)
        if key not in host:
            cg, ag = sample["banks_g"][i % COPIES]
            cd, ad = sample["banks_d"][i % COPIES]
            host[key] = (cg[e].cpu().numpy(), ag[e].cpu().numpy(), cd[e].cpu().numpy(),
                         ad[e].cpu().numpy())
        return host[key]

    steps = range(len(sample["ids"]))
    rates, done_all, blas = [], 0, []
    with threadpool_limits(limits=threads):
        blas = [{k: d.get(k) for k in ("internal_api", "version", "num_threads",
                                        "threading_layer")}
                for d in threadpool_info() if d.get("user_api") == "blas"]
        for _ in range(runs):
            done, nbytes, elapsed = 0, 0, 0.0
            for i in steps:
                ids = sample["ids"][i]
                active = sorted(set(ids.reshape(-1).tolist()))
                h = {e: fetch(i, e) for e in active}
                t0 = time.perf_counter()
                wg = {e: oracle.nf4_decode(h[e][0], h[e][1]) for e in active}
                wd = {e: oracle.nf4_decode(h[e][2], h[e][3]) for e in active}
                oracle.grouped_gemm(x_bits, lambda e: wg[e], ids, E)
                oracle.grouped_gemm(xd_bits, lambda e: wd[e], ids.reshape(-1, 1), E)
                elapsed += time.perf_counter() - t0
                done += 1
                d = len(active)
                nbytes += (d * (nf4_expert_bytes(Ng, Kg) + nf4_expert_bytes(Nd, Kd))
                           + Kg * 2 + topk * Ng * 2 + topk * Kd * 2 + topk * Nd * 2)
                if elapsed >= budget_s / runs:
                    break
            rates.append(nbytes / elapsed / 1e9)
            done_all += done
    used = max([b["num_threads"] or 1 for b in blas] + [1])
    return {"value": float(np.median(rates)), "unit": "GB/s", "cores": used, "kind": "oracle",
            "runs_gbs": [round(r, 4) for r in rates],
            "cpu_model": cpu_info(), "affinity_cpus": affinity, "blas": blas,
            "sample": f"median of {runs} runs over {done_all} timed decode steps in all (M=1, "
                      f"gate_up + down, 8 experts each, about {budget_s / runs:.0f} s per run): "
                      f"NumPy NF4 decode of the active experts + float64 grouped matmul, BLAS "
                      f"on {used} threads"}


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
    """Floats rounded to 4 decimals, recursively."""
    if isinstance(d, float):
        return round(d, 4)
    if isinstance(d, dict):
        return {k: r4(v) for k, v in d.items()}
    if isinstance(d, (list, tuple)):
        return [r4(v) for v in d]
    return d


LEGS = ("decode", "decode_m4", "mx_decode", "controls", "prefill", "mx_prefill",
        "mx_prefill_scaled", "layer_decode", "layer_prefill", "mx_layer_decode",
        "mx_layer_prefill", "host_stream", "dequant", "dgrad", "mx_dgrad", "mfma")


def run_legs(dev, args, legs):
    """The named legs only (for profiler runs), one JSON object of results."""
    out = {}
    st, wu, ps, pw = args.steps, args.warmup, args.prefill_steps, args.prefill_warmup
    for leg in legs:
        log("[bench] leg", leg)
        if leg == "decode":
            out[leg] = decode_nf4(dev, st, wu, M=1)[0]
        elif leg == "decode_m4":
            out[leg] = decode_nf4(dev, st, wu, M=4)[0]
        elif leg == "mx_decode":
            out[leg] = decode_mx(dev, st, wu)
        elif leg == "controls":
            out[leg] = controls(dev, [16 << 20, 140_000_000])
        elif leg == "prefill":
            out[leg] = prefill(dev, ps, pw, "nf4")
        elif leg == "mx_prefill":
            out[leg] = prefill(dev, ps, pw, "mx")
        elif leg == "mx_prefill_scaled":
            out[leg] = prefill_mx_scaled(dev, ps, pw)
        elif leg == "layer_decode":
            out[leg] = decode_layer_nf4(dev, st, wu)
        elif leg == "layer_prefill":
            out[leg] = prefill_layer_nf4(dev, ps, pw)
        elif leg == "mx_layer_decode":
            out[leg] = decode_layer_mx(dev, st, wu)
        elif leg == "mx_layer_prefill":
            out[leg] = prefill_layer_mx(dev, ps, pw)
        elif leg == "host_stream":
            out[leg] = host_stream(dev, min(st, 50), min(wu, 5))
        elif leg == "dequant":
            out[leg] = dequant_baseline(dev, st, wu)
        elif leg == "dgrad":
            out[leg] = dgrad(dev, ps, pw)
        elif leg == "mx_dgrad":
            out[leg] = dgrad(dev, ps, pw, "mx")
        elif leg == "mfma":
            out[leg] = mfma_rates(dev)
        else:
            sys.exit(f"unknown leg {leg}; choose from {','.join(LEGS)}")
        log("[bench]", leg, r4(out[leg]))
    print(json.dumps(r4(out)), flush=True)


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
    ap.add_argument("--legs", default=None,
                    help="profiling runs: comma-separated subset of " + ",".join(LEGS) +
                         "; runs only those legs and prints their results (not the bench line)")
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
    if args.legs:
        run_legs(dev, args, args.legs.split(","))
        return

    log("[bench] nf4 decode M=1")
    dec, sample = decode_nf4(dev, args.steps, args.warmup, M=1)
    log("[bench]", r4(dec))
    log("[bench] mxfp4 decode M=1")
    dmx = decode_mx(dev, args.steps, args.warmup)
    log("[bench]", r4(dmx))
    # the four one-token launches: (name, algorithmic bytes, device us)
    launches = [("nf4_gate_up", dec["gate_up_bytes_per_launch"], dec["gate_up_us"]),
                ("nf4_down", dec["down_bytes_per_launch"], dec["down_us"]),
                ("mxfp4_gate_up", dmx["gate_up_bytes_per_launch"], dmx["gate_up_us"]),
                ("mxfp4_down", dmx["down_bytes_per_launch"], dmx["down_us"])]
    log("[bench] controls")
    ctl = controls(dev, [int(b) for _, b, _ in launches] + [140_000_000])
    log("[bench] controls", ctl)
    t0, bw = fit_line([b for _, b, _ in launches], [u for _, _, u in launches])
    decode_fit = {
        "model": "t = t0 + bytes / bw_eff, least squares over the four one-token GEMV launches",
        "t0_us": t0, "bw_eff_gbs": bw, "bw_eff_frac_hbm": bw / HBM_PEAK_GBS,
        "launches": [{"kernel": n, "bytes": round(b), "us": u,
                      "gbs": b / (u * 1e-6) / 1e9, "frac_hbm": b / (u * 1e-6) / 1e9 / HBM_PEAK_GBS,
                      "control_us": c["us"], "frac_of_control": c["us"] / u}
                     for (n, b, u), c in zip(launches, ctl["stream"])]}
    log("[bench] decode fit", decode_fit)
    log("[bench] mfma rates")
    rates = mfma_rates(dev)
    log("[bench] mfma rates", rates)
    log("[bench] nf4 prefill M=4096")
    pre = prefill(dev, args.prefill_steps, args.prefill_warmup, "nf4")
    log("[bench]", r4(pre))
    extra = {}
    if not args.quick:
        log("[bench] nf4 decode M=4")
        d4, _ = decode_nf4(dev, args.steps, args.warmup, M=4)
        extra["nf4_decode_m4"] = {"workload": "qwen3-30b-a3b nf4 decode gemv M=4", **d4,
                                  "gate_up_frac_hbm": d4["gate_up_gbs"] / HBM_PEAK_GBS}
        extra["mxfp4_decode_m1"] = dmx
        log("[bench] mxfp4 prefill M=2048")
        mp = prefill(dev, args.prefill_steps, args.prefill_warmup, "mx")
        mp["workload"] = "gpt-oss-20b mxfp4 prefill M=2048 top-4 (bf16 MFMA on exact decode)"
        mp["gate_up_frac_bf16_peak"] = mp["gate_up_tflops"] / BF16_PEAK_TFLOPS
        mp["gate_up_frac_fp4_peak"] = mp["gate_up_tflops"] / FP4_PEAK_TFLOPS
        extra["mxfp4_prefill_m2048"] = mp
        log("[bench] mxfp4 prefill M=2048 (block-scaled fp4 instruction)")
        extra["mxfp4_prefill_m2048_scaled"] = prefill_mx_scaled(dev, args.prefill_steps,
                                                                args.prefill_warmup)
        log("[bench]", r4(extra["mxfp4_prefill_m2048_scaled"]))
        log("[bench] nf4 moe layer decode M=1")
        extra["nf4_moe_layer_decode_m1"] = decode_layer_nf4(dev, args.steps, args.warmup)
        log("[bench] nf4 moe layer prefill M=4096")
        extra["nf4_moe_layer_prefill_m4096"] = prefill_layer_nf4(dev, args.prefill_steps,
                                                                 args.prefill_warmup)
        log("[bench] mxfp4 moe layer decode M=1")
        extra["mxfp4_moe_layer_decode_m1"] = decode_layer_mx(dev, args.steps, args.warmup)
        log("[bench] mxfp4 moe layer prefill M=2048")
        extra["mxfp4_moe_layer_prefill_m2048"] = prefill_layer_mx(dev, args.prefill_steps,
                                                                  args.prefill_warmup)
        log("[bench] nf4 decode from pinned host memory")
        extra["nf4_decode_m1_host_streamed"] = host_stream(dev, min(args.steps, 50),
                                                           min(args.warmup, 5))
        log("[bench] dequantize-then-GEMM comparator")
        dq = dequant_baseline(dev, args.steps, args.warmup)
        dq["workload"] = ("qwen3-30b-a3b nf4, dequantize-then-GEMM (decode to a bf16 copy, then "
                          "hipBLASLt per expert): decode M=1 and prefill M=4096 Zipf, the same "
                          "workloads as the headline and prefill legs")
        dq["fused_speedup_decode_m1"] = dq["decode_m1_ms_per_step"] / dec["ms_per_step"]
        dq["fused_speedup_prefill_m4096"] = dq["prefill_m4096_ms_per_step"] / pre["ms_per_step"]
        extra["dequant_then_gemm"] = dq
        log("[bench]", r4(dq))
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
                     "controls": ctl,
                     "decode_fit": decode_fit},
        "mfma_rates": rates,
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
    print(json.dumps(r4(line)), flush=True)


if __name__ == "__main__":
    main()
