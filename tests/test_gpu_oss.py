"""gpt-oss's gated unit fused into the MXFP4 gate_up products, on the GPU
against the float64 oracle (oracle.gate_up_swiglu_oss): the decode GEMV
(in-wave and LDS-reduced rows) and the prefill GEMM on the block-scaled fp4
instruction.  Activations are also drawn 8x larger so that many gate and up
values pass the clamps; one-hot probes, whose products are exact, pin the
unit itself to one bf16 ulp; ragged tiles, tile edges, dropped pairs and
the gpt-oss-20b shapes (sampled experts).  Then the MXFP4 decode down GEMV
with the router-weighted combine fused, and whole gpt-oss decode layers."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, assert_rows, assert_slices, bf16_bits,
                              bf16_to_host_f32, device, packed_mx_bank, same_codes, say, to_dev,
                              to_dev_bf16, unpermute_split)

pytestmark = pytest.mark.gpu


def _ref(x, W, ids, E):
    return oracle.gate_up_swiglu_oss(x, W, ids, E)


def _clamp_share(x, W, ids, E):
    """Share of gate values above the clamp in the reference products (the
    tests with scaled activations need the clamps in play)."""
    h = oracle.grouped_gemm(x, W, np.where(ids >= E, -1, ids), E)
    return float(np.mean(h[:, 0::2] > oracle.OSS_LIMIT))


def _gemm_act(x_bits, blocks, scales, ids, E, dev):
    route = gq.gq_route_sort(to_dev(ids.astype(np.int32), dev), E)
    split = gq.gq_act_split_e4m3(to_dev_bf16(x_bits, dev))
    out = gq.gq_mxfp4_grouped_gemm_scaled_swiglu(split, blocks, scales, route)
    torch.cuda.synchronize()
    return out


# ---- decode GEMV ---------------------------------------------------------------
@pytest.mark.parametrize("K,rows,xstd", [(96, 1, 1.0), (96, 3, 8.0), (2880, 2, 1.0),
                                         (2880, 3, 8.0), (1024, 2, 8.0)])
def test_gemv_swiglu_oss_small(K, rows, xstd):
    """K = 96 and 1024: a row's segments inside one wave; K = 2880: rows
    reduced through LDS.  A dropped slot gives a zero row."""
    dev = device()
    g = np.random.default_rng(K * 10 + rows)
    E, I, topk = 4, 80, 2
    blocks, scales = packed_mx_bank(g, E, 2 * I, K)
    W = LazyDecoded("mx", blocks, scales)
    x = wl.draw_bf16(g, (rows, K), std=xstd)
    ids = wl.route_uniform(g, rows, E, topk)
    if rows > 1:
        ids[1, 0] = -1
    say("gemv swiglu oss", K, rows, xstd)
    act = gq.gq_mxfp4_grouped_gemv_swiglu(to_dev_bf16(x, dev), to_dev(blocks, dev),
                                          to_dev(scales, dev), to_dev(ids, dev))
    torch.cuda.synchronize()
    got, ref = bf16_to_host_f32(act), _ref(x, W, ids, E)
    if xstd > 1 and K >= 1024:
        assert _clamp_share(x, W, ids, E) > 0.05
    assert_slices(got, ref, ids, E)
    assert_rows(got, ref)


def test_gemv_swiglu_oss_gptoss():
    """gpt-oss-20b decode: one token, top-4 of 32 experts, gate_up
    [5760, 2880] (gate row 2j, up row 2j + 1)."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N2, K = wl.GPTOSS["gate_up"]
    blocks, scales = wl.random_mxfp4_bank(E, N2, K, dev, seed=4300)
    g = wl.rng(wl.CFG_GPTOSS, 60)
    x = wl.draw_bf16(g, (1, K), std=4.0)
    ids = wl.route_uniform(g, 1, E, topk)
    say("gemv swiglu oss gpt-oss")
    act = gq.gq_mxfp4_grouped_gemv_swiglu(to_dev_bf16(x, dev), blocks, scales, to_dev(ids, dev))
    torch.cuda.synchronize()
    W = LazyDecoded("mx", blocks.cpu().numpy(), scales.cpu().numpy())
    got, ref = bf16_to_host_f32(act), _ref(x, W, ids, E)
    assert_slices(got, ref, ids, E)
    assert_rows(got, ref)


# ---- prefill GEMM on the block-scaled instruction --------------------------------
@pytest.mark.parametrize("N2,K,xstd", [(288, 1056, 1.0), (288, 1056, 8.0), (544, 2880, 8.0),
                                       (256, 64, 1.0)])
def test_gemm_scaled_swiglu_oss_ragged(N2, K, xstd):
    """Skewed routing over several 256-row tiles, I = 144 and 272 ending
    inside a 128-output tile, K = 1056 with a half-filled last step,
    dropped and out-of-range ids."""
    dev = device()
    g = np.random.default_rng(N2 + 5 * K + int(xstd))
    E, M, topk = 6, 700, 2
    blocks, scales = packed_mx_bank(g, E, N2, K)
    W = LazyDecoded("mx", blocks, scales)
    ids = wl.route_zipf(g, M, E, topk, s=2.5)
    ids[g.random(ids.shape) < 0.02] = -1
    ids[:, 1][ids[:, 1] == 4] = E
    x = wl.draw_bf16(g, (M, K), std=xstd)
    say("mx8 swiglu ragged", N2, K, xstd)
    got = bf16_to_host_f32(_gemm_act(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev))
    ref = _ref(x, W, np.where(ids >= E, -1, ids), E)
    if xstd > 1:
        assert _clamp_share(x, W, ids, E) > 0.05
    assert got.shape == (M * topk, N2 // 2)
    assert_slices(got, ref, ids, E)
    assert_rows(got, ref)
    assert not got[(ids.reshape(-1) < 0) | (ids.reshape(-1) >= E)].any()


def test_gemm_scaled_swiglu_oss_tile_edges():
    """Segments of 128/129 (4 vs 8 sub-tiles), 161, 224, 256/257, 1, 33 rows,
    an empty expert and dropped pairs, in flatten mode."""
    dev = device()
    g = np.random.default_rng(77)
    sizes = [128, 129, 161, 224, 256, 257, 1, 33, 0]
    E, N2, K = len(sizes), 320, 2880
    ids = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in enumerate(sizes)]
                         + [np.full(5, -1, dtype=np.int32)])
    ids = g.permutation(ids).reshape(-1, 1)
    blocks, scales = packed_mx_bank(g, E, N2, K)
    W = LazyDecoded("mx", blocks, scales)
    x = wl.draw_bf16(g, (ids.shape[0], K), std=4.0)
    say("mx8 swiglu tile edges")
    got = bf16_to_host_f32(_gemm_act(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev))
    ref = _ref(x, W, ids, E)
    assert_slices(got, ref, ids, E)
    assert_rows(got, ref)
    assert not got[ids.reshape(-1) < 0].any()


def _ulp_close(a_bits, b_bits):
    """bf16 patterns equal or one ulp apart (same sign; +-0 equal)."""
    a = np.asarray(a_bits, np.int64)
    b = np.asarray(b_bits, np.int64)
    a = np.where(a == 0x8000, 0, a)
    b = np.where(b == 0x8000, 0, b)
    same_sign = (a >> 15) == (b >> 15)
    return bool(np.all((a == b) | (same_sign & (np.abs(a - b) <= 1))))


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_one_hot_probe(path):
    """x = c * e_k makes each gate and up value an exact multiple of one
    decoded weight (c = 1, 256, 2048: inside and far beyond the clamps), so
    the only rounding left is the unit's float32 arithmetic and the bf16
    output: every output within one bf16 ulp of the float64 oracle."""
    dev = device()
    g = np.random.default_rng(19)
    E, I, K = 2, 96, 1056
    blocks, scales = packed_mx_bank(g, E, 2 * I, K)
    W = LazyDecoded("mx", blocks, scales)
    ks = np.array([0, 31, 32, 517, K - 1])
    cs = np.array([0x3F80, 0x4380, 0x4500], dtype=np.uint16)      # 1, 256, 2048
    x = np.zeros((len(ks) * len(cs), K), dtype=np.uint16)
    for i, (k, c) in enumerate([(k, c) for k in ks for c in cs]):
        x[i, k] = c
    ids = np.stack([np.zeros(len(x)), np.ones(len(x))], axis=1).astype(np.int32)
    say("oss one-hot", path)
    if path == "gemv":
        outs = []
        for r0 in range(0, len(x), 8):                   # <= 8 rows per GEMV call
            a = gq.gq_mxfp4_grouped_gemv_swiglu(to_dev_bf16(x[r0:r0 + 8], dev),
                                                to_dev(blocks, dev), to_dev(scales, dev),
                                                to_dev(ids[r0:r0 + 8], dev))
            outs.append(bf16_bits(a))
        torch.cuda.synchronize()
        got = np.concatenate(outs)
    else:
        got = bf16_bits(_gemm_act(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev))
    ref = _ref(x, W, ids, E)
    assert np.mean(np.abs(oracle.grouped_gemm(x, W, ids, E)[:, 0::2]) > 7) > 0.2
    want = oracle.f32_to_bf16_rne(ref.astype(np.float32))
    assert _ulp_close(got, want)


def test_gemm_scaled_swiglu_oss_gptoss_full():
    """gpt-oss-20b prefill gate_up at M = 2048, top-4 of 32 experts, with
    29 dropped pairs; three sampled experts checked per slice and per row."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N2, K = wl.GPTOSS["gate_up"]
    M = 2048
    blocks, scales = wl.random_mxfp4_bank(E, N2, K, dev, seed=4400)
    ids = wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), M, E, topk).copy()
    drop = np.random.default_rng(44).choice(ids.size, 29, replace=False)
    ids.reshape(-1)[drop] = -1
    x = wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X), (M, K), std=4.0)
    say("mx8 swiglu gpt-oss full")
    got = bf16_to_host_f32(_gemm_act(x, blocks, scales, ids, E, dev))
    W = LazyDecoded("mx", blocks.cpu().numpy(), scales.cpu().numpy())
    check = [0, 13, 31]
    ref = _ref(x, W, np.where(np.isin(ids, check), ids, -1), E)
    assert_slices(got, ref, ids, E, experts=check)
    rows = np.nonzero(np.isin(ids.reshape(-1), check))[0]
    assert_rows(got[rows], ref[rows], what="sampled experts")
    assert not got[drop].any()


# ---- the gated unit written as the next product's e4m3 split ----------------------
def _split_pair(x_bits, blocks, scales, ids, E, dev):
    """(fused split, split of the bf16 result) of the same gate_up product."""
    route = gq.gq_route_sort(to_dev(ids.astype(np.int32), dev), E)
    xs = gq.gq_act_split_e4m3(to_dev_bf16(x_bits, dev))
    fused = gq.gq_mxfp4_grouped_gemm_scaled_swiglu_split(xs, blocks, scales, route)
    act = gq.gq_mxfp4_grouped_gemm_scaled_swiglu(xs, blocks, scales, route)
    after = gq.gq_act_split_e4m3(act)
    torch.cuda.synchronize()
    return fused, after, act


def _assert_same_bytes(fused, after):
    for a, b, what in zip(fused, after, ("codes", "scales")):
        diff = (a != b).nonzero()
        assert diff.shape[0] == 0, (what, diff[:5].tolist())


@pytest.mark.parametrize("N2,K,xstd", [(256, 1056, 1.0), (640, 2880, 8.0), (384, 64, 8.0)])
def test_gemm_scaled_swiglu_split_equals_split_of_result(N2, K, xstd):
    """The fused split's code and scale bytes equal gq_act_split_e4m3 of the
    bf16 result, over skewed routing on several tiles, I = 128, 320 and 192
    (a last 128-output tile half full), clamped values, dropped and
    out-of-range ids (their rows: zero codes, zero scale bytes)."""
    dev = device()
    g = np.random.default_rng(3 * N2 + K + int(xstd))
    E, M, topk = 6, 700, 2
    blocks, scales = packed_mx_bank(g, E, N2, K)
    ids = wl.route_zipf(g, M, E, topk, s=2.5)
    ids[g.random(ids.shape) < 0.02] = -1
    ids[:, 1][ids[:, 1] == 4] = E
    x = wl.draw_bf16(g, (M, K), std=xstd)
    say("mx8 swiglu split", N2, K, xstd)
    fused, after, act = _split_pair(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev)
    assert tuple(fused[0].shape) == (M * topk, N2) and tuple(fused[1].shape) == (M * topk, N2 // 32)
    _assert_same_bytes(fused, after)
    dropped = torch.from_numpy((ids.reshape(-1) < 0) | (ids.reshape(-1) >= E)).to(dev)
    assert int(dropped.sum()) > 0
    assert not fused[0][dropped].any() and not fused[1][dropped].any()
    # and against the oracle's split of the bf16 result
    hi, lo, sh, sl = unpermute_split(fused[0].cpu().numpy(), fused[1].cpu().numpy(), N2 // 2)
    rhi, rlo, rsh, rsl = oracle.act_split_e4m3(bf16_bits(act))
    assert np.array_equal(sh, rsh) and np.array_equal(sl, rsl)
    assert same_codes(hi, rhi) and same_codes(lo, rlo)


def test_gemm_scaled_swiglu_split_tile_edges():
    """Segments of 128/129, 161, 224, 256/257, 1, 33 rows, an empty expert
    and dropped pairs in flatten mode: bytes equal the split of the result."""
    dev = device()
    g = np.random.default_rng(78)
    sizes = [128, 129, 161, 224, 256, 257, 1, 33, 0]
    E, N2, K = len(sizes), 384, 2880
    ids = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in enumerate(sizes)]
                         + [np.full(5, -1, dtype=np.int32)])
    ids = g.permutation(ids).reshape(-1, 1)
    blocks, scales = packed_mx_bank(g, E, N2, K)
    x = wl.draw_bf16(g, (ids.shape[0], K), std=4.0)
    say("mx8 swiglu split tile edges")
    fused, after, _ = _split_pair(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev)
    _assert_same_bytes(fused, after)


def test_gemm_scaled_swiglu_split_gptoss_full():
    """gpt-oss-20b gate_up at M = 2048, top-4 of 32, with dropped pairs:
    every code and scale byte of the fused split equals the split of the
    bf16 result (both on the device; the bf16 result is checked against the
    oracle by test_gemm_scaled_swiglu_oss_gptoss_full)."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N2, K = wl.GPTOSS["gate_up"]
    M = 2048
    blocks, scales = wl.random_mxfp4_bank(E, N2, K, dev, seed=4401)
    ids = wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), M, E, topk).copy()
    drop = np.random.default_rng(45).choice(ids.size, 29, replace=False)
    ids.reshape(-1)[drop] = -1
    x = wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X), (M, K), std=4.0)
    say("mx8 swiglu split gpt-oss full")
    fused, after, _ = _split_pair(x, blocks, scales, ids, E, dev)
    _assert_same_bytes(fused, after)
    d = torch.from_numpy(drop).to(dev)
    assert not fused[0][d].any() and not fused[1][d].any()


# ---- decode down projection with the router-weighted combine -------------------
@pytest.mark.parametrize("rows,topk,I,weighted", [(1, 4, 96, True), (3, 2, 2880, False),
                                                 (1, 4, 2880, True), (8, 4, 2880, True),
                                                 (2, 8, 4096, True), (16, 4, 1024, True)])
def test_down_combine_mx_small(rows, topk, I, weighted):
    """MXFP4 down GEMV + combine: in-wave rows (I <= 2048) and two segments
    per lane (I = 2880, 4096), one and two pairs per wave, a dropped slot."""
    dev = device()
    g = np.random.default_rng(rows * 100 + topk * 10 + I)
    E, H = 9, 200
    blocks, scales = packed_mx_bank(g, E, H, I)
    act = wl.draw_bf16(g, (rows * topk, I))
    ids = wl.route_uniform(g, rows, E, topk)
    if rows > 2:
        ids[2, 1] = -1
    w = wl.router_weights(g, rows, topk) if weighted else None
    say("mx down combine", rows, topk, I, weighted)
    y = gq.gq_mxfp4_grouped_gemv_down_combine(to_dev_bf16(act, dev), to_dev(blocks, dev),
                                              to_dev(scales, dev), to_dev(ids, dev),
                                              None if w is None else to_dev(w, dev))
    torch.cuda.synchronize()
    ref = oracle.down_combine(act, LazyDecoded("mx", blocks, scales), ids, E, w)
    assert_rows(bf16_to_host_f32(y), ref)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_layer_gptoss(M):
    """One gpt-oss-20b decode MoE layer: gate_up GEMV with the gated unit,
    then down GEMV + router-weighted combine; each launch against the oracle
    on its own input, and the float64 chain end to end."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    (N2, K), (H, I) = wl.GPTOSS["gate_up"], wl.GPTOSS["down"]
    bg, sg = wl.random_mxfp4_bank(E, N2, K, dev, seed=4500 + M)
    bd, sd = wl.random_mxfp4_bank(E, H, I, dev, seed=4600 + M)
    g = wl.rng(wl.CFG_GPTOSS, 70 + M)
    x = wl.draw_bf16(g, (M, K), std=4.0)
    ids = wl.route_uniform(g, M, E, topk)
    w = wl.router_weights(g, M, topk)
    say("decode layer gpt-oss", M)
    t_ids = to_dev(ids, dev)
    act = gq.gq_mxfp4_grouped_gemv_swiglu(to_dev_bf16(x, dev), bg, sg, t_ids)
    y = gq.gq_mxfp4_grouped_gemv_down_combine(act, bd, sd, t_ids, to_dev(w, dev))
    torch.cuda.synchronize()
    Wg = LazyDecoded("mx", bg.cpu().numpy(), sg.cpu().numpy())
    Wd = LazyDecoded("mx", bd.cpu().numpy(), sd.cpu().numpy())
    assert_rows(bf16_to_host_f32(act), _ref(x, Wg, ids, E), what="gate_up")
    act_bits = bf16_bits(act)
    assert_rows(bf16_to_host_f32(y), oracle.down_combine(act_bits, Wd, ids, E, w), what="down")
    act64 = _ref(x, Wg, ids, E)
    y64 = oracle.combine(np.stack([act64[p] @ Wd(ids.reshape(-1)[p]).astype(np.float64).T
                                   for p in range(M * topk)]), topk, w)
    assert_rows(bf16_to_host_f32(y), y64, tol=8e-3, what="end to end")
