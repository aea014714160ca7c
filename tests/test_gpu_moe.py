"""MoE-layer epilogues on the GPU against the float64 oracle: SwiGLU fused
into the gate_up GEMV and GEMM, the decode down GEMV with the router-
weighted combine fused in, and the prefill combine kernel."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, assert_rows, assert_slices, bf16_to_host_f32, device,
                              packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _rel_rows_ok(got, ref, tol=oracle.REL_L2_TOL):
    """Per-row relative L2 <= tol; rows whose reference is exactly zero are zero."""
    for i in range(ref.shape[0]):
        nr = np.linalg.norm(ref[i])
        if nr == 0.0:
            assert not np.any(got[i]), f"row {i} should be zero"
        else:
            err = np.linalg.norm(got[i] - ref[i]) / nr
            assert err <= tol, f"row {i}: rel-L2 {err}"


# ---- SwiGLU ------------------------------------------------------------------
@pytest.mark.parametrize("K,rows", [(512, 1), (512, 3), (4096, 2), (192, 2)])
def test_gemv_swiglu_small(K, rows):
    """K = 512 and 192: in-wave rows; K = 4096: rows reduced through LDS."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 400 + K + rows)
    E, I, topk = 4, 96, 2
    codes, absmax = packed_nf4_bank(g, E, 2 * I, K)
    x = wl.draw_bf16(g, (rows, K))
    ids = wl.route_uniform(g, rows, E, topk)
    if rows > 1:
        ids[1, 0] = -1                                  # dropped slot: zero row
    say("gemv swiglu", K, rows)
    act = gq.gq_nf4_grouped_gemv_swiglu(to_dev_bf16(x, dev), to_dev(codes, dev),
                                        to_dev(absmax, dev), to_dev(ids, dev))
    torch.cuda.synchronize()
    ref = oracle.gate_up_swiglu(x, LazyDecoded("nf4", codes, absmax), ids, E)
    assert_slices(bf16_to_host_f32(act), ref, ids, E)


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_swiglu_qwen(M):
    dev = device()
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    N2, K = wl.QWEN["gate_up"]
    codes, absmax = wl.random_nf4_bank(E, N2, K, dev, seed=7000 + M)
    g = wl.rng(wl.CFG_QWEN_DECODE, 40 + M)
    x = wl.draw_bf16(g, (M, K))
    ids = wl.route_uniform(g, M, E, topk)
    say("gemv swiglu qwen", M)
    act = gq.gq_nf4_grouped_gemv_swiglu(to_dev_bf16(x, dev), codes, absmax, to_dev(ids, dev))
    torch.cuda.synchronize()
    W = LazyDecoded("nf4", codes.cpu().numpy(), absmax.cpu().numpy())
    ref = oracle.gate_up_swiglu(x, W, ids, E)
    assert_slices(bf16_to_host_f32(act), ref, ids, E)


@pytest.mark.parametrize("E,I,K,M,topk", [(6, 160, 384, 300, 2), (3, 96, 256, 70, 3),
                                          (6, 160, 1024, 300, 2), (3, 96, 1152, 70, 3)])
def test_gemm_swiglu_small(E, I, K, M, topk):
    """Several row tiles, a ragged last tile; I = 96 and I = 160 leave a
    partial output tile (64 outputs per tile below K = 1024, 128 from there)."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 500 + I + M)
    codes, absmax = packed_nf4_bank(g, E, 2 * I, K)
    x = wl.draw_bf16(g, (M, K))
    ids = wl.route_zipf(g, M, E, topk, s=1.5)
    ids[g.random(ids.shape) < 0.03] = -1
    say("gemm swiglu", E, I, K, M, topk)
    route = gq.gq_route_sort(to_dev(ids, dev), E)
    act = gq.gq_nf4_grouped_gemm_swiglu(to_dev_bf16(x, dev), to_dev(codes, dev),
                                        to_dev(absmax, dev), route)
    torch.cuda.synchronize()
    ref = oracle.gate_up_swiglu(x, LazyDecoded("nf4", codes, absmax), ids, E)
    assert_slices(bf16_to_host_f32(act), ref, ids, E)


def test_gemm_swiglu_qwen_prefill():
    """The bench's prefill launch (4096 tokens, Zipf top-8); three experts checked."""
    dev = device()
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    N2, K = wl.QWEN["gate_up"]
    M = 4096
    codes, absmax = wl.random_nf4_bank(E, N2, K, dev, seed=7100)
    ids = wl.route_zipf(wl.rng(wl.CFG_QWEN_PREFILL, wl.S_ROUTE), M, E, topk)
    x = wl.draw_bf16(wl.rng(wl.CFG_QWEN_PREFILL, wl.S_X), (M, K))
    say("gemm swiglu qwen prefill")
    route = gq.gq_route_sort(to_dev(ids, dev), E)
    act = gq.gq_nf4_grouped_gemm_swiglu(to_dev_bf16(x, dev), codes, absmax, route)
    torch.cuda.synchronize()
    W = LazyDecoded("nf4", codes.cpu().numpy(), absmax.cpu().numpy())
    check = [0, 40, 127]
    keep = np.isin(ids.reshape(-1), check)
    ref = oracle.gate_up_swiglu(x, W, np.where(np.isin(ids, check), ids, -1), E)
    got = bf16_to_host_f32(act)
    assert_slices(got[keep], ref[keep], ids.reshape(-1)[keep], E)
    assert_rows(got[keep], ref[keep], what="sampled experts")


def test_swiglu_matches_unfused_path():
    """Fused SwiGLU vs the plain GEMV output put through the same formula on
    the host: the two agree to bf16 rounding of the intermediate."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 600)
    E, I, K, topk = 4, 128, 512, 2
    codes, absmax = packed_nf4_bank(g, E, 2 * I, K)
    x = wl.draw_bf16(g, (1, K))
    ids = wl.route_uniform(g, 1, E, topk)
    args = (to_dev_bf16(x, dev), to_dev(codes, dev), to_dev(absmax, dev), to_dev(ids, dev))
    say("swiglu vs unfused")
    fused = bf16_to_host_f32(gq.gq_nf4_grouped_gemv_swiglu(*args))
    plain = bf16_to_host_f32(gq.gq_nf4_grouped_gemv(*args)).astype(np.float64)
    torch.cuda.synchronize()
    _rel_rows_ok(fused, oracle.swiglu(plain), tol=8e-3)


# ---- down projection + combine ------------------------------------------------
@pytest.mark.parametrize("rows,topk,I,weighted", [(1, 2, 128, True), (3, 2, 128, False),
                                                 (4, 4, 192, True), (2, 8, 2048, True),
                                                 (5, 8, 768, False), (8, 8, 2048, True),
                                                 (1, 8, 4096, True), (4, 8, 3072, False)])
def test_down_combine_small(rows, topk, I, weighted):
    """One to four pairs per wave, lane groups of 4..64 lanes, up to 64 pairs;
    I = 3072 and 4096: two segments per lane (one and two pairs per wave)."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 700 + rows * 10 + topk + I)
    E, H = 9, 200
    codes, absmax = packed_nf4_bank(g, E, H, I)
    act = wl.draw_bf16(g, (rows * topk, I))
    ids = wl.route_uniform(g, rows, E, topk)
    if rows > 2:
        ids[2, 1] = -1                                  # dropped slot contributes 0
    w = wl.router_weights(g, rows, topk) if weighted else None
    say("down combine", rows, topk, I, weighted)
    y = gq.gq_nf4_grouped_gemv_down_combine(to_dev_bf16(act, dev), to_dev(codes, dev),
                                            to_dev(absmax, dev), to_dev(ids, dev),
                                            None if w is None else to_dev(w, dev))
    torch.cuda.synchronize()
    ref = oracle.down_combine(act, LazyDecoded("nf4", codes, absmax), ids, E, w)
    _rel_rows_ok(bf16_to_host_f32(y), ref)


@pytest.mark.parametrize("M", [1, 4])
def test_decode_layer_qwen(M):
    """One decode MoE layer on the Qwen3 shapes: SwiGLU gate_up GEMV then
    down GEMV + combine, against the oracle fed the GPU's bf16 activations
    (each launch checked on its own input) and the end-to-end float64 chain."""
    dev = device()
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    (N2, K), (H, I) = wl.QWEN["gate_up"], wl.QWEN["down"]
    cg, ag = wl.random_nf4_bank(E, N2, K, dev, seed=7200 + M)
    cd, ad = wl.random_nf4_bank(E, H, I, dev, seed=7300 + M)
    g = wl.rng(wl.CFG_QWEN_DECODE, 60 + M)
    x = wl.draw_bf16(g, (M, K))
    ids = wl.route_uniform(g, M, E, topk)
    w = wl.router_weights(g, M, topk)
    say("decode layer qwen", M)
    t_ids = to_dev(ids, dev)
    act = gq.gq_nf4_grouped_gemv_swiglu(to_dev_bf16(x, dev), cg, ag, t_ids)
    y = gq.gq_nf4_grouped_gemv_down_combine(act, cd, ad, t_ids, to_dev(w, dev))
    torch.cuda.synchronize()
    Wd = LazyDecoded("nf4", cd.cpu().numpy(), ad.cpu().numpy())
    act_bits = act.view(torch.int16).cpu().numpy().view(np.uint16)
    _rel_rows_ok(bf16_to_host_f32(y), oracle.down_combine(act_bits, Wd, ids, E, w))
    Wg = LazyDecoded("nf4", cg.cpu().numpy(), ag.cpu().numpy())
    act64 = oracle.gate_up_swiglu(x, Wg, ids, E)
    y64 = oracle.combine(np.stack([act64[p] @ Wd(ids.reshape(-1)[p]).astype(np.float64).T
                                   for p in range(M * topk)]), topk, w)
    _rel_rows_ok(bf16_to_host_f32(y), y64, tol=8e-3)


# ---- prefill combine ------------------------------------------------------------
@pytest.mark.parametrize("rows,topk,H,weighted", [(5, 8, 2048, True), (300, 4, 2880, False),
                                                 (1, 1, 8, True)])
def test_moe_combine(rows, topk, H, weighted):
    dev = device()
    g = wl.rng(wl.CFG_TINY, 800 + rows + H)
    yp = wl.draw_bf16(g, (rows * topk, H))
    w = wl.router_weights(g, rows, topk) if weighted else None
    say("moe combine", rows, topk, H, weighted)
    y = gq.gq_moe_combine(to_dev_bf16(yp, dev), topk, None if w is None else to_dev(w, dev))
    torch.cuda.synchronize()
    ref = oracle.combine(oracle.bf16_to_f32(yp).astype(np.float64), topk, w)
    _rel_rows_ok(bf16_to_host_f32(y), ref)
