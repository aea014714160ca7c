"""NF4 input gradient on the GPU against the float64 oracle: small and
ragged multi-tile cases with dropped pairs and a partial column tile,
one-hot probes bit for bit, the full Qwen3-30B-A3B backward (sampled
experts), determinism."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, plus_zero, packed_mx_bank, assert_rows,
                              assert_slices, bf16_bits, bf16_to_host_f32, device,
                              packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _dgrad(dy_bits, codes, absmax, pe, E, dev):
    dy = to_dev_bf16(dy_bits, dev)
    route = gq.gq_route_sort(to_dev(pe.astype(np.int32).reshape(-1, 1), dev), E)
    out = gq.gq_nf4_grouped_dgrad(dy, codes, absmax, route)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("E,N,K,P", [(4, 256, 512, 64), (6, 320, 704, 900),
                                     (4, 1024, 512, 600), (6, 1088, 704, 900)])
def test_small_and_ragged(E, N, K, P):
    """Several row tiles per expert with a ragged tail, dropped pairs, and a
    partial column tile (K = 704: 5.5 tiles of 128 columns)."""
    dev = device()
    g = np.random.default_rng(N + K)
    codes, absmax = packed_nf4_bank(g, E, N, K)
    W = LazyDecoded("nf4", codes, absmax)
    pe = wl.route_zipf(g, P, E, 1, s=2.0).reshape(-1)
    pe[g.random(P) < 0.03] = -1
    dy = wl.draw_bf16(g, (P, N))
    say("dgrad", E, N, K, P)
    out = _dgrad(dy, to_dev(codes, dev), to_dev(absmax, dev), pe, E, dev)
    ref = oracle.grouped_dgrad(dy, W, pe, E)
    assert_slices(bf16_to_host_f32(out), ref, pe, E)


def test_tile_boundaries():
    """Expert segments on and next to the 256-row tile edges (512, 256, 257,
    255 and 1 pairs), an empty expert and dropped pairs."""
    dev = device()
    g = np.random.default_rng(23)
    E, N, K = 7, 192, 320
    sizes = [512, 256, 257, 1, 0, 255, 0]
    pe = np.concatenate([np.full(n, e, dtype=np.int32) for e, n in enumerate(sizes)]
                        + [np.full(9, -1, dtype=np.int32)])
    pe = g.permutation(pe)
    codes, absmax = packed_nf4_bank(g, E, N, K)
    W = LazyDecoded("nf4", codes, absmax)
    dy = wl.draw_bf16(g, (pe.shape[0], N))
    say("dgrad tile boundaries")
    out = _dgrad(dy, to_dev(codes, dev), to_dev(absmax, dev), pe, E, dev)
    assert_slices(bf16_to_host_f32(out), oracle.grouped_dgrad(dy, W, pe, E), pe, E)


@pytest.mark.parametrize("N,K", [(128, 256), (1024, 320)])
def test_one_hot_probe_is_bit_exact(N, K):
    """dY = e_n makes dX row p the decoded weight row W[n, :] rounded once
    (K = 320 leaves a 64-column tile)."""
    dev = device()
    g = np.random.default_rng(6)
    E = 2
    codes, absmax = packed_nf4_bank(g, E, N, K)
    W = LazyDecoded("nf4", codes, absmax)
    ns = np.array(sorted({0, 1, 63, 64, N // 2 + 9, N - 1}))
    dy = np.zeros((2 * len(ns), N), dtype=np.uint16)
    pe = np.zeros(2 * len(ns), dtype=np.int32)
    for i, n in enumerate(ns):
        dy[2 * i, n] = dy[2 * i + 1, n] = 0x3F80
        pe[2 * i + 1] = 1
    say("dgrad one-hot", N, K)
    out = bf16_bits(_dgrad(dy, to_dev(codes, dev), to_dev(absmax, dev), pe, E, dev))
    for i, n in enumerate(ns):
        for s in range(2):
            want = oracle.f32_to_bf16_rne(W(s)[n])
            assert np.array_equal(plus_zero(out[2 * i + s]), plus_zero(want)), (n, s)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_qwen_dgrad_full_shapes(proj):
    """2048 tokens x top-8 = 16384 pairs over 128 experts: the bench's launch.
    Checked on three experts, every row."""
    dev = device()
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    N, K = wl.QWEN[proj]
    codes, absmax = wl.random_nf4_bank(E, N, K, dev, seed=5000 + N)
    pe = wl.route_uniform(wl.rng(wl.CFG_QWEN_DGRAD, wl.S_ROUTE), 2048, E, topk).reshape(-1)
    dy = wl.draw_bf16(wl.rng(wl.CFG_QWEN_DGRAD, wl.S_DOWN_IN), (pe.size, N))
    say("dgrad qwen", proj)
    out = _dgrad(dy, codes, absmax, pe, E, dev)
    W = LazyDecoded("nf4", codes.cpu().numpy(), absmax.cpu().numpy())
    check = [0, 64, 127]
    ref = oracle.grouped_dgrad(dy, W, np.where(np.isin(pe, check), pe, -1), E)
    yg = bf16_to_host_f32(out)
    assert_slices(yg, ref, pe, E, experts=check)
    rows = np.nonzero(np.isin(pe, check))[0]
    assert_rows(yg[rows], ref[rows], what="sampled experts")


def test_deterministic():
    dev = device()
    g = np.random.default_rng(12)
    E, N, K, P = 8, 256, 384, 1000
    codes, absmax = packed_nf4_bank(g, E, N, K)
    pe = g.integers(0, E, P)
    dy = wl.draw_bf16(g, (P, N))
    say("dgrad determinism")
    a = _dgrad(dy, to_dev(codes, dev), to_dev(absmax, dev), pe, E, dev)
    b = _dgrad(dy, to_dev(codes, dev), to_dev(absmax, dev), pe, E, dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- MXFP4 -----------------------------------------------------------------
def _dgrad_mx(dy_bits, blocks, scales, pe, E, dev):
    dy = to_dev_bf16(dy_bits, dev)
    route = gq.gq_route_sort(to_dev(pe.astype(np.int32).reshape(-1, 1), dev), E)
    out = gq.gq_mxfp4_grouped_dgrad(dy, blocks, scales, route)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("E,N,K,P", [(4, 128, 256, 64), (5, 192, 352, 700), (3, 320, 2880, 300),
                                     (3, 1024, 2880, 300), (4, 1152, 352, 500)])
def test_mx_small_and_ragged(E, N, K, P):
    """K = 352 and 2880 leave a partial 128-column tile (K % 64 == 32 for
    352); N = 1024, 1152 give 16-18 contraction steps."""
    dev = device()
    g = np.random.default_rng(N + 3 * K)
    blocks, scales = packed_mx_bank(g, E, N, K)
    W = LazyDecoded("mx", blocks, scales)
    pe = wl.route_zipf(g, P, E, 1, s=2.0).reshape(-1)
    pe[g.random(P) < 0.03] = -1
    dy = wl.draw_bf16(g, (P, N))
    say("mx dgrad", E, N, K, P)
    out = _dgrad_mx(dy, to_dev(blocks, dev), to_dev(scales, dev), pe, E, dev)
    ref = oracle.grouped_dgrad(dy, W, pe, E)
    assert_slices(bf16_to_host_f32(out), ref, pe, E)
    dropped = pe < 0
    assert not bf16_bits(out)[dropped].any() or not dropped.any()


@pytest.mark.parametrize("N,K", [(128, 224), (1024, 288)])
def test_mx_one_hot_probe_is_bit_exact(N, K):
    """dY = e_n makes dX row p the decoded MXFP4 weight row W[n, :] (exact in
    bf16); K = 288 leaves a 32-column tile."""
    dev = device()
    g = np.random.default_rng(16)
    E = 2
    blocks, scales = packed_mx_bank(g, E, N, K)
    W = LazyDecoded("mx", blocks, scales)
    ns = np.array(sorted({0, 1, 63, 64, N // 2 + 9, N - 1}))
    dy = np.zeros((2 * len(ns), N), dtype=np.uint16)
    pe = np.zeros(2 * len(ns), dtype=np.int32)
    for i, n in enumerate(ns):
        dy[2 * i, n] = dy[2 * i + 1, n] = 0x3F80
        pe[2 * i + 1] = 1
    say("mx dgrad one-hot", N, K)
    out = bf16_bits(_dgrad_mx(dy, to_dev(blocks, dev), to_dev(scales, dev), pe, E, dev))
    for i, n in enumerate(ns):
        for s in range(2):
            want = oracle.f32_to_bf16_rne(W(s)[n])
            assert np.array_equal(plus_zero(out[2 * i + s]), plus_zero(want)), (n, s)


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_gptoss_mx_dgrad_full_shapes(proj):
    """gpt-oss-20b shapes, 2048 tokens x top-4 = 8192 pairs over 32 experts.
    Checked on three experts, every row."""
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N, K = wl.GPTOSS[proj]
    blocks, scales = wl.random_mxfp4_bank(E, N, K, dev, seed=6000 + N)
    pe = wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), 2048, E, topk).reshape(-1)
    dy = wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_DOWN_IN), (pe.size, N))
    say("mx dgrad gpt-oss", proj)
    out = _dgrad_mx(dy, blocks, scales, pe, E, dev)
    W = LazyDecoded("mx", blocks.cpu().numpy(), scales.cpu().numpy())
    check = [0, 17, 31]
    ref = oracle.grouped_dgrad(dy, W, np.where(np.isin(pe, check), pe, -1), E)
    yg = bf16_to_host_f32(out)
    assert_slices(yg, ref, pe, E, experts=check)
    rows = np.nonzero(np.isin(pe, check))[0]
    assert_rows(yg[rows], ref[rows], what="sampled experts")


def test_mx_deterministic():
    dev = device()
    g = np.random.default_rng(13)
    E, N, K, P = 8, 256, 416, 1000
    blocks, scales = packed_mx_bank(g, E, N, K)
    pe = g.integers(0, E, P)
    dy = wl.draw_bf16(g, (P, N))
    say("mx dgrad determinism")
    a = _dgrad_mx(dy, to_dev(blocks, dev), to_dev(scales, dev), pe, E, dev)
    b = _dgrad_mx(dy, to_dev(blocks, dev), to_dev(scales, dev), pe, E, dev)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
