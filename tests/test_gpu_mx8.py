"""MXFP4 on the block-scaled fp4 matrix instruction, on the GPU against the
oracle: the two-term e4m3 activation split bit for bit (codes and scale
bytes), then the grouped GEMM against the float64 W4A16 product (per-expert
and per-row relative L2 <= 4e-3) and against the product of the split
activations, one-hot probes bit for bit, ragged multi-tile segments, tile
edges, a K tail, dropped pairs, pair scales, the gpt-oss-20b M = 2048
launches (sampled experts), determinism."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, assert_rows, assert_slices, bf16_bits,
                              bf16_to_host_f32, device, packed_mx_bank, plus_zero, same_codes, say,
                              to_dev, to_dev_bf16, unpermute_split)

pytestmark = pytest.mark.gpu


def _split(x_bits, dev):
    codes, scales = gq.gq_act_split_e4m3(to_dev_bf16(x_bits, dev))
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


@pytest.mark.parametrize("rows,K", [(7, 64), (33, 2880), (5, 544), (64, 2048), (3, 32)])
def test_split_bit_exact(rows, K):
    """Codes and scale bytes equal the oracle's; K = 544 and 32 leave a
    half-filled last step whose pad must be zero."""
    dev = device()
    g = np.random.default_rng(rows * 1000 + K)
    x = wl.draw_bf16(g, (rows, K))
    x[0, :32] = 0                                         # all-zero block
    if rows > 2:
        x[1, :] = wl.draw_bf16(g, (1, K), std=1e-39)      # bf16 subnormal values
        x[2, :32] = wl.draw_bf16(g, (1, 32), std=1e4)[0]  # wide dynamic range in one row
        x[2, 1] = 0x3F80                                  # 1.0 next to 1e4-scale values
    say("split", rows, K)
    codes, scales = _split(x, dev)
    hi, lo, sh, sl = unpermute_split(codes, scales, K)
    rhi, rlo, rsh, rsl = oracle.act_split_e4m3(x)
    assert np.array_equal(sh, rsh) and np.array_equal(sl, rsl)
    assert same_codes(hi, rhi) and same_codes(lo, rlo)
    kp = codes.shape[1] // 2
    if kp > K:                                            # pad block: zeros, scale 0
        c = codes.reshape(rows, kp // 64, 2, 2, 2, 16)
        assert not c[:, -1, :, :, 1, :].any()
        assert not scales.reshape(rows, kp // 64, 2, 2)[:, -1, 1, :].any()


def _gemm(x_bits, blocks, scales, ids, E, dev, pair_scale=None):
    x = to_dev_bf16(x_bits, dev) if isinstance(x_bits, np.ndarray) else x_bits
    route = gq.gq_route_sort(to_dev(ids.astype(np.int32), dev), E)
    sc = None if pair_scale is None else to_dev(pair_scale.astype(np.float32).reshape(-1), dev)
    split = gq.gq_act_split_e4m3(x)
    out = gq.gq_mxfp4_grouped_gemm_scaled(split, blocks, scales, route, pair_scale=sc)
    torch.cuda.synchronize()
    return out


def _split_value_bits(x_bits):
    """The activations the split represents, as float64 (for the tighter
    check against the split product)."""
    return oracle.act_split_value(*oracle.act_split_e4m3(x_bits))


def _split_ref(x_bits, W, ids, E, pair_scale=None):
    """float64 product of the split activations (what the instruction
    computes, up to float32 accumulation)."""
    xs = _split_value_bits(x_bits)
    ids = np.asarray(ids).astype(np.int64)
    rows, topk = ids.shape
    flat = ids.reshape(-1)
    out = None
    for e in range(E):
        pairs = np.nonzero(flat == e)[0]
        if len(pairs) == 0:
            continue
        w = W(e).astype(np.float64)
        if out is None:
            out = np.zeros((rows * topk, w.shape[0]))
        out[pairs] = xs[pairs // topk] @ w.T
    if pair_scale is not None:
        out *= np.asarray(pair_scale, np.float32).reshape(-1).astype(np.float64)[:, None]
    return out


@pytest.mark.parametrize("N,K", [(288, 1056), (160, 1120), (544, 2048), (320, 544), (256, 64)])
def test_ragged_multi_tile(N, K):
    """Skewed routing (one expert over several 256-row tiles, others short
    or empty), N ending inside a 256-column tile, K = 1056, 1120, 544 with a
    half-filled last step, dropped and out-of-range ids, pair scales."""
    dev = device()
    g = np.random.default_rng(N + 7 * K)
    E, M, topk = 6, 700, 2
    blocks, scales = packed_mx_bank(g, E, N, K)
    W = LazyDecoded("mx", blocks, scales)
    ids = wl.route_zipf(g, M, E, topk, s=2.5)
    ids[g.random(ids.shape) < 0.02] = -1
    ids[:, 1][ids[:, 1] == 4] = E
    x = wl.draw_bf16(g, (M, K))
    sc = wl.router_weights(g, M, topk)
    say("mx8 ragged", N, K)
    out = _gemm(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev, sc)
    got = bf16_to_host_f32(out)
    ref = oracle.grouped_gemm(x, W, ids, E, pair_scale=sc)
    assert_slices(got, ref, ids, E)
    assert_rows(got, ref, what="vs W4A16")
    # against the split product: only float32 accumulation and the output rounding
    assert_rows(got, _split_ref(x, W, ids, E, sc), tol=2.5e-3, what="vs split product")


@pytest.mark.parametrize("K,N", [(1056, 288), (2880, 320)])
def test_tile_edges(K, N):
    """Segments of 128/129 rows (4 vs 8 sub-tiles), 161, 192, 224 (6 and 7
    active sub-tiles), 256/257 (a one-row tail tile), 384/385, 1, 32, 33, an
    empty expert and dropped pairs, in flatten mode with pair scales."""
    dev = device()
    g = np.random.default_rng(K + 3 * N)
    sizes = [128, 129, 161, 192, 224, 256, 257, 384, 385, 1, 32, 33, 0]
    E = len(sizes)
    ids = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in enumerate(sizes)]
                         + [np.full(7, -1, dtype=np.int32)])
    ids = g.permutation(ids).reshape(-1, 1)
    blocks, scales = packed_mx_bank(g, E, N, K)
    W = LazyDecoded("mx", blocks, scales)
    x = wl.draw_bf16(g, (ids.shape[0], K))
    sc = g.uniform(0.5, 1.5, size=ids.shape).astype(np.float32)
    say("mx8 tile edges", K, N)
    out = _gemm(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev, sc)
    got = bf16_to_host_f32(out)
    ref = oracle.grouped_gemm(x, W, ids, E, pair_scale=sc)
    assert_slices(got, ref, ids, E)
    assert_rows(got, ref, what="vs W4A16")
    assert not got[ids.reshape(-1) < 0].any()


@pytest.mark.parametrize("K", [256, 1056])
def test_one_hot_probe_is_bit_exact(K):
    """x = e_k splits into hi = 256 (e4m3 0x78) with scale 2^-8 and lo = 0,
    so the output row is the decoded weight column, bit for bit (K = 1056:
    the last step is half filled)."""
    dev = device()
    g = np.random.default_rng(11)
    E, N = 2, 128
    blocks, scales = packed_mx_bank(g, E, N, K)
    W = LazyDecoded("mx", blocks, scales)
    ks = np.array(sorted({0, 1, 15, 16, 31, 32, 47, 48, 63, 64, 100, K // 2 + 7, K - 33,
                          K - 32, K - 1}))
    x = np.zeros((len(ks), K), dtype=np.uint16)
    x[np.arange(len(ks)), ks] = 0x3F80
    ids = np.stack([np.zeros(len(ks)), np.ones(len(ks))], axis=1).astype(np.int32)
    say("mx8 one-hot", K)
    out = bf16_bits(_gemm(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev))
    for t, k in enumerate(ks):
        for s in range(2):
            want = oracle.f32_to_bf16_rne(W(s)[:, k])
            assert np.array_equal(plus_zero(out[2 * t + s]), plus_zero(want)), (t, s, k)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_gptoss_full_shapes(proj):
    """gpt-oss-20b at M = 2048, top-4 over 32 experts: gate_up [5760, 2880]
    in gather mode, down [2880, 2880] in flatten mode with router-weight
    scales, as the bench launches them; three sampled experts checked per
    slice and per row, dropped pairs zero."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N, K = wl.GPTOSS[proj]
    M = 2048
    blocks, scales = wl.random_mxfp4_bank(E, N, K, dev, seed=4100 if proj == "gate_up" else 4101)
    ids = wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), M, E, topk)
    sc = None
    if proj == "down":
        sc = wl.router_weights(wl.rng(wl.CFG_GPTOSS, wl.S_LOGITS), M, topk).reshape(-1, 1)
        ids = ids.reshape(-1, 1)
    ids = ids.copy()
    drop = np.random.default_rng(43).choice(ids.size, 29, replace=False)
    ids.reshape(-1)[drop] = -1
    x = wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X if proj == "gate_up" else wl.S_DOWN_IN),
                     (ids.shape[0], K))
    say("mx8 gpt-oss", proj)
    out = _gemm(x, blocks, scales, ids, E, dev, sc)
    W = LazyDecoded("mx", blocks.cpu().numpy(), scales.cpu().numpy())
    check = [0, 17, 31]
    ref = oracle.grouped_gemm(x, W, np.where(np.isin(ids, check), ids, -1), E, pair_scale=sc)
    got = bf16_to_host_f32(out)
    assert_slices(got, ref, ids, E, experts=check)
    rows = np.nonzero(np.isin(ids.reshape(-1), check))[0]
    assert_rows(got[rows], ref[rows], what="sampled experts")
    assert not got[drop].any()


def test_deterministic():
    dev = device()
    g = np.random.default_rng(21)
    E, N, K = 5, 256, 1024
    blocks, scales = packed_mx_bank(g, E, N, K)
    ids = wl.route_zipf(g, 900, E, 2)
    x = wl.draw_bf16(g, (900, K))
    say("mx8 determinism")
    a = _gemm(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev)
    b = _gemm(x, to_dev(blocks, dev), to_dev(scales, dev), ids, E, dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
