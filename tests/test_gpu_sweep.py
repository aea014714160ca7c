"""Seeded random shapes through the prefill GEMM (NF4, MXFP4, SwiGLU), the
input gradient and the decode launches against the float64 oracle: expert counts, row counts
per expert (so tiles of every size class: <= 128 rows, 129..255, full,
several), column counts ending inside a tile, K on both sides of the
kernel switch (MXFP4 with a half step), dropped ids, pair scales and
strided activations.  Each case names itself before its launch."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, assert_slices, bf16_to_host_f32, device,
                              packed_mx_bank, packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu

N_CASES = 36


def _case(seed):
    g = np.random.default_rng(9000 + seed)
    fmt = ["nf4", "mx", "glu"][seed % 3]
    E = int(g.integers(2, 9))
    kq = 64 if fmt != "mx" else 32
    K = int(g.choice([kq * int(g.integers(4, 15)), kq * int(g.integers(16, 40))]))
    N = (64 if fmt == "glu" else 32) * int(g.integers(2, 15))
    M = int(g.integers(1, 400))
    topk = int(g.integers(1, min(E, 4) + 1))
    return g, fmt, E, N, K, M, topk


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_forward(seed):
    dev = device()
    g, fmt, E, N, K, M, topk = _case(seed)
    bank = packed_mx_bank(g, E, N, K) if fmt == "mx" else packed_nf4_bank(g, E, N, K)
    W = LazyDecoded("mx" if fmt == "mx" else "nf4", *bank)
    ids = wl.route_zipf(g, M, E, topk, s=float(g.uniform(0.5, 2.5)))
    ids[g.random(ids.shape) < 0.05] = -1
    pad = 8 * int(g.integers(0, 3))
    full = wl.draw_bf16(g, (M, K + pad))
    xh = np.ascontiguousarray(full[:, :K])
    x = to_dev_bf16(full, dev)[:, :K]
    sc = None if fmt == "glu" else wl.router_weights(g, M, topk)
    say("sweep forward", seed, fmt, E, N, K, M, topk, pad)
    route = gq.gq_route_sort(to_dev(ids, dev), E)
    if fmt == "glu":
        out = gq.gq_nf4_grouped_gemm_swiglu(x, to_dev(bank[0], dev), to_dev(bank[1], dev), route)
        ref = oracle.gate_up_swiglu(xh, W, ids, E)
    else:
        fn = gq.gq_nf4_grouped_gemm if fmt == "nf4" else gq.gq_mxfp4_grouped_gemm
        out = fn(x, to_dev(bank[0], dev), to_dev(bank[1], dev), route,
                 pair_scale=to_dev(sc.reshape(-1), dev))
        ref = oracle.grouped_gemm(xh, W, ids, E, pair_scale=sc)
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(out), ref, ids, E)


@pytest.mark.parametrize("seed", range(N_CASES // 2))
def test_random_dgrad(seed):
    dev = device()
    g = np.random.default_rng(9500 + seed)
    fmt = "nf4" if seed % 2 == 0 else "mx"
    E = int(g.integers(2, 7))
    N = 64 * int(g.integers(2, 12))                 # the contraction: a multiple of 64
    K = 32 * int(g.integers(2, 20))
    if fmt == "nf4":
        K = 64 * (K // 64 or 1)
    P = int(g.integers(1, 700))
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    pe = wl.route_zipf(g, P, E, 1, s=float(g.uniform(0.5, 2.5))).reshape(-1)
    pe[g.random(P) < 0.05] = -1
    dy = wl.draw_bf16(g, (P, N))
    say("sweep dgrad", seed, fmt, E, N, K, P)
    route = gq.gq_route_sort(to_dev(pe.astype(np.int32).reshape(-1, 1), dev), E)
    fn = gq.gq_nf4_grouped_dgrad if fmt == "nf4" else gq.gq_mxfp4_grouped_dgrad
    dx = fn(to_dev_bf16(dy, dev), to_dev(bank[0], dev), to_dev(bank[1], dev), route)
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(dx), oracle.grouped_dgrad(dy, W, pe, E), pe, E)


def _wide_bits(g, rows, cols, dev):
    """bf16 [rows, cols] device view with a random row padding, and its host bits."""
    pad = 8 * int(g.integers(0, 3))
    full = wl.draw_bf16(g, (rows, cols + pad))
    return to_dev_bf16(full, dev)[:, :cols], np.ascontiguousarray(full[:, :cols])


def _rows_close(got, ref, tol=oracle.REL_L2_TOL):
    for i in range(ref.shape[0]):
        nr = np.linalg.norm(ref[i])
        if nr == 0.0:
            assert not np.any(got[i]), i
        else:
            assert np.linalg.norm(got[i] - ref[i]) / nr <= tol, i


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_decode(seed):
    """Decode launches: NF4 / MXFP4 GEMV (gather or flatten mode, pair
    scales), the SwiGLU GEMV and the down GEMV with the combine fused."""
    dev = device()
    g = np.random.default_rng(9800 + seed)
    kind = ["nf4", "mx", "glu", "down"][seed % 4]
    E = int(g.integers(1, 10))
    rows = int(g.integers(1, 9))
    topk = int(g.integers(1, min(E, 8) + 1))
    if kind == "down":
        topk = min(topk, 64 // rows)
        K = 64 * int(g.integers(1, 33))                    # I <= 2048
    elif kind == "mx":
        K = 32 * int(g.integers(1, 257))                   # <= 8192
    else:
        K = 64 * int(g.integers(1, 129))
    N = 2 * int(g.integers(1, 400)) if kind == "glu" else int(g.integers(1, 700))
    bank = packed_mx_bank(g, E, N, K) if kind == "mx" else packed_nf4_bank(g, E, N, K)
    W = LazyDecoded("mx" if kind == "mx" else "nf4", *bank)
    a, b = to_dev(bank[0], dev), to_dev(bank[1], dev)
    ids = wl.route_uniform(g, rows, E, topk) if g.random() < 0.5 else \
        g.integers(0, E, size=(rows, topk)).astype(np.int32)  # repeated experts too
    ids[g.random(ids.shape) < 0.1] = -1
    say("sweep decode", seed, kind, E, N, K, rows, topk)
    if kind == "down":
        act, acth = _wide_bits(g, rows * topk, K, dev)
        w = wl.router_weights(g, rows, topk) if g.random() < 0.5 else None
        y = gq.gq_nf4_grouped_gemv_down_combine(act, a, b, to_dev(ids, dev),
                                                None if w is None else to_dev(w, dev))
        torch.cuda.synchronize()
        _rows_close(bf16_to_host_f32(y), oracle.down_combine(acth, W, ids, E, w))
        return
    flatten = kind != "glu" and g.random() < 0.3
    if flatten:                                            # one input row per pair
        x, xh = _wide_bits(g, rows * topk, K, dev)
        ids = ids.reshape(-1, 1)
    else:
        x, xh = _wide_bits(g, rows, K, dev)
    if kind == "glu":
        out = gq.gq_nf4_grouped_gemv_swiglu(x, a, b, to_dev(ids, dev))
        ref = oracle.gate_up_swiglu(xh, W, ids, E)
    else:
        sc = wl.router_weights(g, ids.shape[0], ids.shape[1]) if g.random() < 0.5 else None
        fn = gq.gq_nf4_grouped_gemv if kind == "nf4" else gq.gq_mxfp4_grouped_gemv
        out = fn(x, a, b, to_dev(ids, dev),
                 pair_scale=None if sc is None else to_dev(sc.reshape(-1), dev))
        ref = oracle.grouped_gemm(xh, W, ids, E, pair_scale=sc)
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(out), ref, ids, E)
