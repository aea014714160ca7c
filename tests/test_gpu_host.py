"""Experts streamed from pinned host memory: the decode GEMV reading its
expert bank over the host link gives the same bits as the device-resident
call on the same bytes, and matches the float64 oracle; NF4 and MXFP4,
small banks and the Qwen3 / gpt-oss one-token shapes."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import (LazyDecoded, assert_rows, bf16_bits, bf16_to_host_f32, device,
                              packed_mx_bank, packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _pinned(a):
    """A new pinned host tensor holding a (numpy array or CPU/device tensor)."""
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a.cpu()
    p = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    p.copy_(t)
    return p


@pytest.mark.parametrize("fmt,K,rows", [("nf4", 512, 1), ("nf4", 4096, 3), ("mx", 2880, 2),
                                        ("mx", 96, 4)])
def test_host_bank_small(fmt, K, rows):
    dev = device()
    g = np.random.default_rng(K + rows + (7 if fmt == "mx" else 0))
    E, N, topk = 6, 320, 2
    if fmt == "nf4":
        a, b = packed_nf4_bank(g, E, N, K)
        host, devc = gq.gq_nf4_grouped_gemv_host, gq.gq_nf4_grouped_gemv
    else:
        a, b = packed_mx_bank(g, E, N, K)
        host, devc = gq.gq_mxfp4_grouped_gemv_host, gq.gq_mxfp4_grouped_gemv
    x = wl.draw_bf16(g, (rows, K))
    ids = wl.route_uniform(g, rows, E, topk)
    if rows > 1:
        ids[1, 1] = -1
    sc = wl.router_weights(g, rows, topk).reshape(-1)
    xd, idd, scd = to_dev_bf16(x, dev), to_dev(ids, dev), to_dev(sc, dev)
    say("host bank", fmt, K, rows)
    y_host = host(xd, _pinned(a), _pinned(b), idd, pair_scale=scd)
    y_dev = devc(xd, to_dev(a, dev), to_dev(b, dev), idd, pair_scale=scd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y_host), bf16_bits(y_dev))
    ref = oracle.grouped_gemm(x, LazyDecoded(fmt, a, b), ids, E, pair_scale=sc)
    assert_rows(bf16_to_host_f32(y_host), ref)


@pytest.mark.parametrize("model", ["qwen", "gptoss"])
def test_host_bank_one_token(model):
    """Qwen3 NF4 gate_up [1536, 2048] top-8 of 128, gpt-oss MXFP4 gate_up
    [5760, 2880] top-4 of 32: host-streamed bits equal the device bits."""
    dev = device()
    if model == "qwen":
        E, topk = wl.QWEN["E"], wl.QWEN["topk"]
        N, K = wl.QWEN["gate_up"]
        a, b = wl.random_nf4_bank(E, N, K, dev, seed=8100)
        host, devc, fmt = gq.gq_nf4_grouped_gemv_host, gq.gq_nf4_grouped_gemv, "nf4"
        g = wl.rng(wl.CFG_QWEN_DECODE, 90)
    else:
        E, topk = wl.GPTOSS["E"], wl.GPTOSS["topk"]
        N, K = wl.GPTOSS["gate_up"]
        a, b = wl.random_mxfp4_bank(E, N, K, dev, seed=8200)
        host, devc, fmt = gq.gq_mxfp4_grouped_gemv_host, gq.gq_mxfp4_grouped_gemv, "mx"
        g = wl.rng(wl.CFG_GPTOSS, 90)
    x = wl.draw_bf16(g, (1, K))
    ids = wl.route_uniform(g, 1, E, topk)
    xd, idd = to_dev_bf16(x, dev), to_dev(ids, dev)
    ah, bh = _pinned(a), _pinned(b)
    say("host bank one token", model)
    y_host = host(xd, ah, bh, idd)
    y_dev = devc(xd, a, b, idd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y_host), bf16_bits(y_dev))
    W = LazyDecoded(fmt, ah.numpy(), bh.numpy())
    assert_rows(bf16_to_host_f32(y_host), oracle.grouped_gemm(x, W, ids, E))


def test_unpinned_bank_is_rejected_before_launch():
    dev = device()
    g = np.random.default_rng(5)
    a, b = packed_nf4_bank(g, 2, 64, 128)
    x = to_dev_bf16(wl.draw_bf16(g, (1, 128)), dev)
    ids = to_dev(np.array([[0, 1]], np.int32), dev)
    with pytest.raises(ValueError):
        gq.gq_nf4_grouped_gemv_host(x, torch.from_numpy(a), torch.from_numpy(b), ids)
