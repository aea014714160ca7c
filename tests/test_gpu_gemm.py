"""Prefill grouped GEMM (NF4 and MXFP4) on the GPU against the float64
oracle: the tiny workload, multi-tile ragged segments with partial column
tiles, a K tail (MXFP4), dropped pairs, pair scales, one-hot probes bit
for bit, the full Qwen3-30B-A3B Zipf prefill and gpt-oss-20b M=2048
launches (sampled experts), determinism."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, plus_zero, assert_rows,
                              assert_slices, bf16_bits, bf16_to_host_f32, device,
                              packed_mx_bank, packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _gemm(fmt, x_bits, a, b, ids, E, dev, scale=None):
    x = to_dev_bf16(x_bits, dev) if isinstance(x_bits, np.ndarray) else x_bits
    t_ids = to_dev(ids.astype(np.int32), dev)
    route = gq.gq_route_sort(t_ids, E)
    t_sc = None if scale is None else to_dev(scale.astype(np.float32).reshape(-1), dev)
    fn = gq.gq_nf4_grouped_gemm if fmt == "nf4" else gq.gq_mxfp4_grouped_gemm
    out = fn(x, a, b, route, pair_scale=t_sc)
    torch.cuda.synchronize()
    return out


def test_tiny_workload():
    """E=4 experts W [256, 512] NF4-packed by the oracle, 16 tokens, top-2."""
    dev = device()
    cfg = wl.TINY
    E, (N, K), topk, M = cfg["E"], cfg["gate_up"], cfg["topk"], cfg["M"]
    w = wl.draw_weights(wl.rng(wl.CFG_TINY, wl.S_W_GATE_UP), E, N, K)
    packed = [oracle.nf4_pack(w[e]) for e in range(E)]
    codes = np.stack([p[0] for p in packed])
    absmax = np.stack([p[1] for p in packed])
    x = wl.draw_bf16(wl.rng(wl.CFG_TINY, wl.S_X), (M, K))
    ids = wl.route_uniform(wl.rng(wl.CFG_TINY, wl.S_ROUTE), M, E, topk)
    scale = wl.router_weights(wl.rng(wl.CFG_TINY, wl.S_LOGITS), M, topk)
    W = LazyDecoded("nf4", codes, absmax)
    for sc in (None, scale):
        say("gemm tiny", sc is not None)
        out = _gemm("nf4", x, to_dev(codes, dev), to_dev(absmax, dev), ids, E, dev, sc)
        assert out.shape == (M * topk, N)
        ref = oracle.grouped_gemm(x, W, ids, E, pair_scale=sc)
        assert_slices(bf16_to_host_f32(out), ref, ids, E)


@pytest.mark.parametrize("fmt,N,K", [("nf4", 320, 768), ("mx", 288, 544), ("mx", 160, 576),
                                     ("nf4", 320, 1088), ("nf4", 544, 1024), ("mx", 288, 1056),
                                     ("mx", 160, 1120)])
def test_ragged_multi_tile(fmt, N, K):
    """Skewed routing: one expert spans several 256-row tiles with a ragged
    tail, others are short or empty; N is not a multiple of the column tile
    (128 for K < 1024, 256 from K = 1024 on, where the other kernel runs);
    MXFP4 K = 544, 1056, 1120 leave a half 64-step; some ids are dropped."""
    dev = device()
    g = np.random.default_rng(N + K)
    E, M, topk = 6, 700, 2
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    ids = wl.route_zipf(g, M, E, topk, s=2.5)
    ids[g.random(ids.shape) < 0.02] = -1                      # dropped pairs
    ids[:, 1][ids[:, 1] == 4] = E                             # out-of-range ids are dropped too
    x = wl.draw_bf16(g, (M, K))
    sc = wl.router_weights(g, M, topk)
    say("gemm ragged", fmt, N, K)
    out = _gemm(fmt, x, to_dev(bank[0], dev), to_dev(bank[1], dev), ids, E, dev, sc)
    ref = oracle.grouped_gemm(x, W, ids, E, pair_scale=sc)
    assert_slices(bf16_to_host_f32(out), ref, ids, E)


@pytest.mark.parametrize("fmt,K", [("nf4", 768), ("mx", 544), ("nf4", 1088), ("mx", 1056)])
def test_tile_boundaries(fmt, K):
    """Expert segments on and next to the 256-row tile edges, in flatten mode
    (one row per pair): 512 rows (two full tiles), 256, 257 (a one-row
    tail tile), 1, 255, an empty expert, and dropped pairs scattered among
    them; both forward kernels (K < 1024 and K >= 1024)."""
    dev = device()
    g = np.random.default_rng(K + 17)
    E, N = 7, 192
    sizes = [512, 256, 257, 1, 0, 255, 0]
    ids = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in enumerate(sizes)]
                         + [np.full(9, -1, dtype=np.int32)])
    ids = g.permutation(ids).reshape(-1, 1)
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    x = wl.draw_bf16(g, (ids.shape[0], K))
    say("gemm tile boundaries", fmt, K)
    out = _gemm(fmt, x, to_dev(bank[0], dev), to_dev(bank[1], dev), ids, E, dev)
    assert_slices(bf16_to_host_f32(out), oracle.grouped_gemm(x, W, ids, E), ids, E)


@pytest.mark.parametrize("fmt,K,N", [("nf4", 1088, 320), ("mx", 1056, 288), ("nf4", 2048, 512)])
def test_narrow_tile_edges(fmt, K, N):
    """K >= 1024: the 256-column kernel runs tiles of at most 128 rows with
    4 sub-tiles per wave (each wave loads its own 32 rows) and longer tiles
    with 8 (8-row groups dealt round-robin to the waves), each specialised
    per count of active 32-row sub-tiles.  Segments of 128 and 129 rows, 384
    and 385 (a full tile then 128 or 129 rows), 161, 192 and 224 (6 and 7
    active sub-tiles), 32, 33, 97 and 1, an empty expert, dropped pairs; N
    ends inside a 256-column tile (a column tile whose last waves own no
    columns)."""
    dev = device()
    g = np.random.default_rng(K + N)
    E = 13
    sizes = [128, 129, 384, 385, 32, 33, 97, 1, 0, 64, 161, 192, 224]
    ids = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in enumerate(sizes)]
                         + [np.full(5, -1, dtype=np.int32)])
    ids = g.permutation(ids).reshape(-1, 1)
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    x = wl.draw_bf16(g, (ids.shape[0], K))
    sc = g.uniform(0.5, 1.5, size=ids.shape).astype(np.float32)
    say("gemm narrow tile edges", fmt, K, N)
    out = _gemm(fmt, x, to_dev(bank[0], dev), to_dev(bank[1], dev), ids, E, dev, sc)
    ref = oracle.grouped_gemm(x, W, ids, E, pair_scale=sc)
    assert_slices(bf16_to_host_f32(out), ref, ids, E)


@pytest.mark.parametrize("fmt,K", [("nf4", 256), ("mx", 256), ("nf4", 1088), ("mx", 1056)])
def test_one_hot_probe_is_bit_exact(fmt, K):
    """A one-hot activation row picks one weight column: the output is the
    decoded weight, bit for bit, in both forward kernels (K = 1056 ends in a
    half-filled MXFP4 step)."""
    dev = device()
    g = np.random.default_rng(5)
    E, N = 2, 128
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    ks = np.array(sorted({0, 1, 31, 32, 63, 64, 100, K // 2 + 7, K - 33, K - 32, K - 1}))
    x = np.zeros((len(ks), K), dtype=np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80
    ids = np.stack([np.zeros(len(ks)), np.ones(len(ks))], axis=1).astype(np.int32)
    say("gemm one-hot", fmt, K)
    out = bf16_bits(_gemm(fmt, x, to_dev(bank[0], dev), to_dev(bank[1], dev), ids, E, dev))
    for t, k in enumerate(ks):
        for s in range(2):
            want = oracle.f32_to_bf16_rne(W(s)[:, k])
            assert np.array_equal(plus_zero(out[2 * t + s]), plus_zero(want)), (t, s, k)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_qwen_prefill_full_shapes(proj):
    """4096 tokens, top-8 Zipf(1.1) routing over 128 experts, router-weight
    scales: the bench's launch.  Checked on the largest, a middle and the
    smallest expert segments (every row of each)."""
    dev = device()
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    N, K = wl.QWEN[proj]
    M = 4096
    codes, absmax = wl.random_nf4_bank(E, N, K, dev, seed=3000 + N)
    ids = wl.route_zipf(wl.rng(wl.CFG_QWEN_PREFILL, wl.S_ROUTE), M, E, topk)
    sc = wl.router_weights(wl.rng(wl.CFG_QWEN_PREFILL, wl.S_LOGITS), M, topk)
    if proj == "down":
        ids, sc = ids.reshape(-1, 1), sc.reshape(-1, 1)
    x = wl.draw_bf16(wl.rng(wl.CFG_QWEN_PREFILL, wl.S_X if proj == "gate_up" else wl.S_DOWN_IN),
                     (ids.shape[0], K))
    say("gemm qwen prefill", proj)
    out = _gemm("nf4", x, codes, absmax, ids, E, dev, sc)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    order = np.argsort(counts)
    check = {int(order[-1]), int(order[E // 2]), int(order[0])}
    W = LazyDecoded("nf4", codes.cpu().numpy(), absmax.cpu().numpy())
    flat = ids.reshape(-1)
    yg = bf16_to_host_f32(out)
    for e in check:
        rows = np.nonzero(flat == e)[0]
        ref = np.zeros((len(rows), N))
        xf = oracle.bf16_to_f32(x).astype(np.float64)
        ref = (xf[rows // ids.shape[1]] @ W(e).astype(np.float64).T) * \
            sc.reshape(-1)[rows].astype(np.float64)[:, None]
        err = np.linalg.norm(yg[rows] - ref) / np.linalg.norm(ref)
        assert err <= oracle.REL_L2_TOL, (e, err)
        assert_rows(yg[rows], ref, what=f"expert {e}")


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_gptoss_prefill_full_shapes(proj):
    """gpt-oss-20b MXFP4 at M = 2048 tokens, top-4 uniform over 32 experts:
    gate_up [5760, 2880] in gather mode and down [2880, 2880] in flatten
    mode (8192 pairs, router-weight scales; its last 64-column tile is the
    guarded one), as the bench launches them.  Three sampled experts are
    checked per slice and per row, and a few dropped pairs must give zero
    rows."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N, K = wl.GPTOSS[proj]
    M = 2048
    blocks, scales = wl.random_mxfp4_bank(E, N, K, dev, seed=4000 if proj == "gate_up" else 4001)
    ids = wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), M, E, topk)
    sc = None
    if proj == "down":
        sc = wl.router_weights(wl.rng(wl.CFG_GPTOSS, wl.S_LOGITS), M, topk).reshape(-1, 1)
        ids = ids.reshape(-1, 1)
    ids = ids.copy()
    drop = np.random.default_rng(41).choice(ids.size, 37, replace=False)
    ids.reshape(-1)[drop] = -1
    x = wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X if proj == "gate_up" else wl.S_DOWN_IN),
                     (ids.shape[0], K))
    say("gemm gpt-oss prefill", proj)
    out = _gemm("mx", x, blocks, scales, ids, E, dev, sc)
    W = LazyDecoded("mx", blocks.cpu().numpy(), scales.cpu().numpy())
    check = [0, 17, 31]
    # the oracle on the sampled experts only (other pairs dropped there)
    ref = oracle.grouped_gemm(x, W, np.where(np.isin(ids, check), ids, -1), E, pair_scale=sc)
    yg = bf16_to_host_f32(out)
    assert_slices(yg, ref, ids, E, experts=check)
    flat = ids.reshape(-1)
    rows = np.nonzero(np.isin(flat, check))[0]
    assert_rows(yg[rows], ref[rows], what="sampled experts")
    assert not np.any(yg[drop]), "dropped pairs must give zero rows"


def test_deterministic_and_route_reuse():
    dev = device()
    g = np.random.default_rng(8)
    E, N, K = 8, 256, 512
    codes, absmax = packed_nf4_bank(g, E, N, K)
    ids = wl.route_zipf(g, 900, E, 2)
    x = wl.draw_bf16(g, (900, K))
    say("gemm determinism")
    a = _gemm("nf4", x, to_dev(codes, dev), to_dev(absmax, dev), ids, E, dev)
    b = _gemm("nf4", x, to_dev(codes, dev), to_dev(absmax, dev), ids, E, dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
