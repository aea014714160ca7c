"""Decode-time grouped GEMV (NF4 and MXFP4) on the GPU against the float64
oracle: per-expert relative L2 <= 4e-3, one-hot probes bit for bit,
dropped pairs, shared experts, pair scales, full Qwen3-30B-A3B and
gpt-oss-20b expert shapes, determinism."""

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


def _run(fmt, x_bits, bank, ids, dev, scale=None):
    x = to_dev_bf16(x_bits, dev)
    a, b = (to_dev(bank[0], dev), to_dev(bank[1], dev))
    t_ids = to_dev(ids.astype(np.int32), dev)
    t_sc = None if scale is None else to_dev(scale.astype(np.float32).reshape(-1), dev)
    fn = gq.gq_nf4_grouped_gemv if fmt == "nf4" else gq.gq_mxfp4_grouped_gemv
    out = fn(x, a, b, t_ids, pair_scale=t_sc)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
@pytest.mark.parametrize("rows", [1, 3, 8])
def test_tiny_gather(fmt, rows):
    dev = device()
    g = wl.rng(wl.CFG_TINY, 100 + rows)
    E, N, K, topk = 4, 256, 512, 2
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    x = wl.draw_bf16(g, (rows, K))
    ids = wl.route_uniform(g, rows, E, topk)
    scale = wl.router_weights(g, rows, topk)
    W = LazyDecoded(fmt, *bank)
    for sc in (None, scale):
        say("gemv tiny", fmt, rows, sc is not None)
        out = _run(fmt, x, bank, ids, dev, sc)
        ref = oracle.grouped_gemm(x, W, ids, E, pair_scale=sc)
        assert_slices(bf16_to_host_f32(out), ref, ids, E)


@pytest.mark.parametrize("fmt,K", [(f, k) for f in ("nf4", "mx")
                                   for k in (64, 128, 256, 1024, 4096, 8192, 192, 96)
                                   if f == "mx" or k % 64 == 0])
def test_k_sweep(fmt, K):
    """Every in-wave reduction width (K/32 segments = 2 .. 64 lanes), the
    cross-wave path (K = 4096, and K = 8192, the longest row the GEMV
    takes), and segment counts that do not divide a wave (K = 96, 192:
    several rows per thread in the cross-wave reduction)."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 300 + K)
    E, N, topk, rows = 3, 160, 2, 2
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    x = wl.draw_bf16(g, (rows, K))
    ids = wl.route_uniform(g, rows, E, topk)
    W = LazyDecoded(fmt, *bank)
    say("gemv k sweep", fmt, K)
    out = _run(fmt, x, bank, ids, dev, None)
    ref = oracle.grouped_gemm(x, W, ids, E)
    assert_slices(bf16_to_host_f32(out), ref, ids, E)


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
def test_shared_experts_dropped_and_flatten(fmt):
    dev = device()
    g = np.random.default_rng(7)
    E, N, K = 3, 192, 320 if fmt == "mx" else 384
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    # 8 tokens, top-4 drawn WITH repeats, plus dropped ids
    ids = g.integers(-1, E + 1, (8, 4)).astype(np.int32)
    x = wl.draw_bf16(g, (8, K))
    say("gemv shared/dropped", fmt)
    out = _run(fmt, x, bank, ids, dev)
    ref = oracle.grouped_gemm(x, W, ids, E)
    assert_slices(bf16_to_host_f32(out), ref, ids, E)
    # flatten mode: one input row per pair, topk = 1, 40 pairs
    fl = ids.reshape(-1, 1)
    xp = wl.draw_bf16(g, (fl.shape[0], K))
    say("gemv flatten", fmt)
    out = _run(fmt, xp, bank, fl, dev)
    ref = oracle.grouped_gemm(xp, W, fl, E)
    assert_slices(bf16_to_host_f32(out), ref, fl, E)


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
@pytest.mark.parametrize("case", ["some", "all"])
def test_dropped_pairs_write_only_their_rows(fmt, case):
    """Dropped ids (-1, which is also the kernel's padding of the routing
    table past the last pair, E, INT32_MAX, -7) give exact zero rows, and no
    store lands outside the [P, N] output: the output sits between two guard
    bands of a sentinel, checked untouched.  Few pairs, so most lanes of the
    routing table are padding."""
    dev = device()
    g = np.random.default_rng(29 if case == "some" else 31)
    E, N, K = 5, 160, 256
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    if case == "some":
        ids = np.array([[2, -1], [-1, 4], [E, 2], [2**31 - 1, -7]], np.int32)
    else:
        ids = np.full((3, 2), -1, np.int32)
    rows, topk = ids.shape
    P, G = rows * topk, 4096
    x = wl.draw_bf16(g, (rows, K))
    sentinel = 0x7A5B
    buf = torch.full((P * N + 2 * G,), sentinel, dtype=torch.int16, device=dev)
    out = buf[G:G + P * N].view(torch.bfloat16).view(P, N)
    fn = gq.gq_nf4_grouped_gemv if fmt == "nf4" else gq.gq_mxfp4_grouped_gemv
    say("gemv dropped guard", fmt, case)
    fn(to_dev_bf16(x, dev), to_dev(bank[0], dev), to_dev(bank[1], dev), to_dev(ids, dev),
       out=out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:G] == sentinel) and np.all(b[G + P * N:] == sentinel)
    got = bf16_to_host_f32(out)
    ref = oracle.grouped_gemm(x, W, ids, E)
    assert_rows(got, ref, what="dropped rows zero, kept rows")
    dropped = ((ids < 0) | (ids >= E)).reshape(-1)
    assert np.all(bf16_bits(out)[dropped] == 0)        # +0.0, not -0.0


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
def test_most_pairs(fmt):
    """The largest routing the GEMV takes: 256 pairs (32 tokens x top-8 in
    gather mode, and the same 256 pairs flattened), experts repeated across
    tokens, a ragged N."""
    dev = device()
    g = np.random.default_rng(11)
    E, N, K = 40, 96 + 32, 256
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    ids = wl.route_uniform(g, 32, E, 8)
    x = wl.draw_bf16(g, (32, K))
    say("gemv 256 pairs gather", fmt)
    out = _run(fmt, x, bank, ids, dev)
    assert_slices(bf16_to_host_f32(out), oracle.grouped_gemm(x, W, ids, E), ids, E)
    fl = ids.reshape(-1, 1)
    xp = wl.draw_bf16(g, (fl.shape[0], K))
    say("gemv 256 pairs flatten", fmt)
    out = _run(fmt, xp, bank, fl, dev)
    assert_slices(bf16_to_host_f32(out), oracle.grouped_gemm(xp, W, fl, E), fl, E)


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
def test_one_hot_probe_is_bit_exact(fmt):
    """x = e_k makes each output the decoded weight W[n, k] itself, rounded
    once to bf16, so the kernel's decode is checked bit for bit."""
    dev = device()
    g = np.random.default_rng(11)
    E, N, K = 2, 128, 256
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    for k in (0, 1, 63, 64, 200, 255):
        x = np.zeros((2, K), dtype=np.uint16)
        x[:, k] = 0x3F80                                   # bf16 1.0
        ids = np.array([[0], [1]], dtype=np.int32)
        say("gemv one-hot", fmt, k)
        out = bf16_bits(_run(fmt, x, bank, ids, dev))
        for p in range(2):
            want = oracle.f32_to_bf16_rne(W(p)[:, k])
            assert np.array_equal(plus_zero(out[p]), plus_zero(want)), (p, k)


QWEN_CASES = [("gate_up", 1), ("down", 1), ("gate_up", 4), ("down", 4)]


@pytest.mark.parametrize("proj,M", QWEN_CASES)
def test_qwen_decode_full_shapes(proj, M):
    """Qwen3-30B-A3B expert bank (E=128) at full size, the bench's launch
    configuration; every active expert checked against the oracle."""
    dev = device()
    E, topk = wl.QWEN["E"], wl.QWEN["topk"]
    N, K = wl.QWEN[proj]
    codes, absmax = wl.random_nf4_bank(E, N, K, dev, seed=1000 + N)
    g = wl.rng(wl.CFG_QWEN_DECODE, wl.S_ROUTE)
    ids = wl.route_uniform(g, M, E, topk)
    if proj == "down":
        ids = ids.reshape(-1, 1)                           # per-pair inputs
    x = wl.draw_bf16(wl.rng(wl.CFG_QWEN_DECODE, wl.S_X), (ids.shape[0], K))
    say("gemv qwen", proj, M)
    out = gq.gq_nf4_grouped_gemv(to_dev_bf16(x, dev), codes, absmax, to_dev(ids, dev))
    torch.cuda.synchronize()
    active = sorted(set(ids.reshape(-1).tolist()))
    cn, an = codes.cpu().numpy(), absmax.cpu().numpy()
    W = LazyDecoded("nf4", cn, an)
    ref = oracle.grouped_gemm(x, W, ids, E)
    worst = assert_slices(bf16_to_host_f32(out), ref, ids, E, experts=active)
    assert worst < 3.5e-3


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_gptoss_decode_full_shapes(proj):
    dev = device()
    E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
    N, K = wl.GPTOSS[proj]
    blocks, scales = wl.random_mxfp4_bank(E, N, K, dev, seed=2000 + N)
    ids = wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), 1, E, topk)
    if proj == "down":
        ids = ids.reshape(-1, 1)
    x = wl.draw_bf16(wl.rng(wl.CFG_GPTOSS, wl.S_X), (ids.shape[0], K))
    say("gemv gpt-oss", proj)
    out = gq.gq_mxfp4_grouped_gemv(to_dev_bf16(x, dev), blocks, scales, to_dev(ids, dev))
    torch.cuda.synchronize()
    W = LazyDecoded("mx", blocks.cpu().numpy(), scales.cpu().numpy())
    ref = oracle.grouped_gemm(x, W, ids, E)
    assert_slices(bf16_to_host_f32(out), ref, ids, E, experts=set(ids.reshape(-1).tolist()))


def test_deterministic():
    dev = device()
    E, N, K = 128, 1536, 2048
    codes, absmax = wl.random_nf4_bank(E, N, K, dev, seed=5)
    ids = to_dev(wl.route_uniform(np.random.default_rng(1), 4, E, 8), dev)
    x = to_dev_bf16(wl.draw_bf16(np.random.default_rng(2), (4, K)), dev)
    say("gemv determinism")
    a = gq.gq_nf4_grouped_gemv(x, codes, absmax, ids)
    b = gq.gq_nf4_grouped_gemv(x, codes, absmax, ids)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
def test_rows_of_x_and_topk_ids_must_agree(fmt):
    """x with more (or fewer) rows than topk_ids is rejected before any
    launch: the kernel would read topk_ids past its end (or leave output
    rows unwritten)."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 900)
    E, N, K = 4, 64, 128
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    a, b = to_dev(bank[0], dev), to_dev(bank[1], dev)
    fn = gq.gq_nf4_grouped_gemv if fmt == "nf4" else gq.gq_mxfp4_grouped_gemv
    ids = to_dev(wl.route_uniform(g, 2, E, 2), dev)
    for rows in (1, 3):
        x = to_dev_bf16(wl.draw_bf16(g, (rows, K)), dev)
        with pytest.raises(ValueError):
            fn(x, a, b, ids)
    if fmt == "nf4":
        x = to_dev_bf16(wl.draw_bf16(g, (3, K)), dev)
        with pytest.raises(ValueError):
            gq.gq_nf4_grouped_gemv_swiglu(x, a, b, ids)
