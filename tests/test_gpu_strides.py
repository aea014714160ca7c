"""Activation / gradient / per-pair inputs that are column slices of wider
tensors (row stride larger than the row length): every entry point that
takes a row stride, against the float64 oracle on the sliced values."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, assert_slices, bf16_to_host_f32, device,
                              packed_mx_bank, packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _wide(g, rows, cols, pad, dev):
    """A bf16 device tensor [rows, cols] viewed out of a [rows, cols + pad]
    one (row stride cols + pad), and the host bits of the view."""
    full = wl.draw_bf16(g, (rows, cols + pad))
    view = to_dev_bf16(full, dev)[:, :cols]
    assert view.stride(0) == cols + pad
    return view, np.ascontiguousarray(full[:, :cols])


def _rows_ok(got, ref, tol=oracle.REL_L2_TOL):
    for i in range(ref.shape[0]):
        nr = np.linalg.norm(ref[i])
        if nr == 0.0:
            assert not np.any(got[i]), i
        else:
            assert np.linalg.norm(got[i] - ref[i]) / nr <= tol, i


@pytest.mark.parametrize("fmt", ["nf4", "mx"])
def test_gemv_and_gemm_strided_x(fmt):
    dev = device()
    g = np.random.default_rng(31)
    E, N, K, topk = 5, 192, 1088 if fmt == "nf4" else 1056, 2
    bank = packed_nf4_bank(g, E, N, K) if fmt == "nf4" else packed_mx_bank(g, E, N, K)
    W = LazyDecoded(fmt, *bank)
    a, b = to_dev(bank[0], dev), to_dev(bank[1], dev)
    gemv = gq.gq_nf4_grouped_gemv if fmt == "nf4" else gq.gq_mxfp4_grouped_gemv
    gemm = gq.gq_nf4_grouped_gemm if fmt == "nf4" else gq.gq_mxfp4_grouped_gemm
    # decode: 3 tokens, row stride K + 64
    x, xh = _wide(g, 3, K, 64, dev)
    ids = wl.route_uniform(g, 3, E, topk)
    say("strided gemv", fmt)
    out = gemv(x, a, b, to_dev(ids, dev))
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(out), oracle.grouped_gemm(xh, W, ids, E), ids, E)
    # prefill: 300 tokens, row stride K + 128 (wide kernel: K >= 1024)
    x, xh = _wide(g, 300, K, 128, dev)
    ids = wl.route_zipf(g, 300, E, topk, s=1.5)
    say("strided gemm", fmt)
    route = gq.gq_route_sort(to_dev(ids, dev), E)
    out = gemm(x, a, b, route)
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(out), oracle.grouped_gemm(xh, W, ids, E), ids, E)


def test_short_k_gemm_and_dgrad_strided():
    dev = device()
    g = np.random.default_rng(37)
    E, N, K = 4, 256, 512
    codes, absmax = packed_nf4_bank(g, E, N, K)
    W = LazyDecoded("nf4", codes, absmax)
    c, am = to_dev(codes, dev), to_dev(absmax, dev)
    # forward on the 256 x 128 kernel (K < 1024), row stride K + 8
    x, xh = _wide(g, 400, K, 8, dev)
    ids = wl.route_zipf(g, 400, E, 2, s=1.5)
    say("strided short-K gemm")
    out = gq.gq_nf4_grouped_gemm(x, c, am, gq.gq_route_sort(to_dev(ids, dev), E))
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(out), oracle.grouped_gemm(xh, W, ids, E), ids, E)
    # input gradient, dY row stride N + 64
    P = 500
    dy, dyh = _wide(g, P, N, 64, dev)
    pe = wl.route_zipf(g, P, E, 1, s=1.5).reshape(-1)
    say("strided dgrad")
    route = gq.gq_route_sort(to_dev(pe.astype(np.int32).reshape(-1, 1), dev), E)
    dx = gq.gq_nf4_grouped_dgrad(dy, c, am, route)
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(dx), oracle.grouped_dgrad(dyh, W, pe, E), pe, E)


def test_down_combine_and_combine_strided():
    dev = device()
    g = np.random.default_rng(41)
    E, H, I, rows, topk = 6, 200, 768, 3, 4
    codes, absmax = packed_nf4_bank(g, E, H, I)
    act, acth = _wide(g, rows * topk, I, 64, dev)
    ids = wl.route_uniform(g, rows, E, topk)
    w = wl.router_weights(g, rows, topk)
    say("strided down combine")
    y = gq.gq_nf4_grouped_gemv_down_combine(act, to_dev(codes, dev), to_dev(absmax, dev),
                                            to_dev(ids, dev), to_dev(w, dev))
    torch.cuda.synchronize()
    _rows_ok(bf16_to_host_f32(y),
             oracle.down_combine(acth, LazyDecoded("nf4", codes, absmax), ids, E, w))
    # prefill combine, per-pair rows of stride H2 + 8
    H2 = 256
    yp, yph = _wide(g, rows * topk, H2, 8, dev)
    say("strided combine")
    y = gq.gq_moe_combine(yp, topk, to_dev(w, dev))
    torch.cuda.synchronize()
    _rows_ok(bf16_to_host_f32(y),
             oracle.combine(oracle.bf16_to_f32(yph).astype(np.float64), topk, w))


def test_swiglu_strided():
    dev = device()
    g = np.random.default_rng(43)
    E, I, topk = 4, 96, 2
    for K, rows, pad in [(512, 2, 24), (1152, 150, 64)]:
        codes, absmax = packed_nf4_bank(g, E, 2 * I, K)
        W = LazyDecoded("nf4", codes, absmax)
        c, am = to_dev(codes, dev), to_dev(absmax, dev)
        x, xh = _wide(g, rows, K, pad, dev)
        ids = wl.route_zipf(g, rows, E, topk, s=1.5)
        say("strided swiglu", K, rows, pad)
        if rows <= 128:
            act = gq.gq_nf4_grouped_gemv_swiglu(x, c, am, to_dev(ids, dev))
        else:
            act = gq.gq_nf4_grouped_gemm_swiglu(x, c, am, gq.gq_route_sort(to_dev(ids, dev), E))
        torch.cuda.synchronize()
        assert_slices(bf16_to_host_f32(act), oracle.gate_up_swiglu(xh, W, ids, E), ids, E)


def test_mx_dgrad_strided():
    dev = device()
    g = np.random.default_rng(47)
    E, N, K, P = 3, 320, 640, 350
    blocks, scales = packed_mx_bank(g, E, N, K)
    dy, dyh = _wide(g, P, N, 40, dev)
    pe = wl.route_zipf(g, P, E, 1, s=1.5).reshape(-1)
    say("strided mx dgrad")
    route = gq.gq_route_sort(to_dev(pe.astype(np.int32).reshape(-1, 1), dev), E)
    dx = gq.gq_mxfp4_grouped_dgrad(dy, to_dev(blocks, dev), to_dev(scales, dev), route)
    torch.cuda.synchronize()
    assert_slices(bf16_to_host_f32(dx),
                  oracle.grouped_dgrad(dyh, LazyDecoded("mx", blocks, scales), pe, E), pe, E)
