"""The dequantize-then-GEMM comparator (bit_grouped_moe_amd.dequant_baseline)
against the float64 oracle, and against the fused kernels on the same
inputs: it must compute the same products for its timings to compare like
with like."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from bit_grouped_moe_amd.dequant_baseline import DequantGemm
from tests.gpu_common import (LazyDecoded, assert_slices, bf16_to_host_f32, device,
                              packed_nf4_bank, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,topk,gather", [(1, 8, True), (3, 2, True), (40, 1, False)])
def test_dequant_gemm_matches_oracle(rows, topk, gather):
    dev = device()
    g = wl.rng(wl.CFG_TINY, 1000 + rows * 10 + topk)
    E, N, K = 9, 192, 512
    codes, absmax = packed_nf4_bank(g, E, N, K)
    ids = wl.route_uniform(g, rows, E, topk)
    ids[rows - 1, 0] = -1                                 # dropped pair: zero row
    n_in = rows if gather else rows * topk
    x = wl.draw_bf16(g, (n_in, K))
    say("dequant gemm", rows, topk, gather)
    dq = DequantGemm(to_dev(codes, dev), to_dev(absmax, dev), max_experts=E)
    out = torch.empty((rows * topk, N), dtype=torch.bfloat16, device=dev)
    tx = to_dev_bf16(x, dev)
    dq.run(tx, dq.plan(ids, gather), out)
    fused = gq.gq_nf4_grouped_gemv(tx, to_dev(codes, dev), to_dev(absmax, dev),
                                   to_dev(ids if gather else ids.reshape(-1, 1), dev))
    torch.cuda.synchronize()
    W = LazyDecoded("nf4", codes, absmax)
    flat_ids = ids if gather else ids.reshape(-1, 1)
    ref = oracle.grouped_gemm(x, W, flat_ids, E)
    got = bf16_to_host_f32(out)
    assert_slices(got, ref, flat_ids, E)
    assert not np.any(got[(rows - 1) * topk])             # the dropped pair stays zero
    # the fused GEMV computes the same products (its weights unrounded)
    f = bf16_to_host_f32(fused)
    for p in range(rows * topk):
        nr = np.linalg.norm(f[p])
        if nr:
            assert np.linalg.norm(got[p] - f[p]) / nr <= 4e-3


def test_dequant_whole_bank_decode():
    """Every expert active: the bank is decoded in one launch; same products."""
    dev = device()
    g = wl.rng(wl.CFG_TINY, 1100)
    E, N, K, M, topk = 4, 128, 256, 64, 2
    codes, absmax = packed_nf4_bank(g, E, N, K)
    ids = wl.route_uniform(g, M, E, topk)
    x = wl.draw_bf16(g, (M, K))
    say("dequant whole bank")
    dq = DequantGemm(to_dev(codes, dev), to_dev(absmax, dev))
    groups = dq.plan(ids, True)
    assert len(groups) == E
    out = torch.empty((M * topk, N), dtype=torch.bfloat16, device=dev)
    dq.run(to_dev_bf16(x, dev), groups, out)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm(x, LazyDecoded("nf4", codes, absmax), ids, E)
    assert_slices(bf16_to_host_f32(out), ref, ids, E)
