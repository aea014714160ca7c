"""Dequantize-then-GEMM comparator for the NF4 expert products.

The standard path the fused kernels are measured against: the routed
experts' packed weights are first decoded to a full bf16 copy (the library's
own decode entry point, gq_nf4_decode, so the weights are bit-identical to
the ones the fused GEMM feeds its matrix cores), then multiplied by the
library GEMM (hipBLASLt, through torch.mm), one expert at a time on that
expert's rows.  Pages: "grouped-nf4-gemm 0.43.0" -- page header (no
full-size bf16 weight copies) and "Try it on your GPU" (packed compute
against dequantize-then-GEMM); "Receipts-driven engineering", "The numbers"
(decode and prefill ratios against the dequant path).

Measurement only: the fused path never calls this module.  The grouping is
taken on the host from the routing (numpy), which the standard path needs
anyway and which this comparator gets outside any timed region.
"""

import numpy as np
import torch

from . import gq_nf4_decode


class DequantGemm:
    """One projection (W [E, N, K] NF4) the standard way.

    ``plan(ids, gather)`` groups the pairs of ``ids`` int32 [rows, topk]
    (numpy) by expert; ``run(x, groups, out)`` decodes every planned expert
    into the bf16 buffer and multiplies x's rows by it (gather: pair p reads
    row p // topk of x; otherwise row p), writing out [rows*topk, N].
    Pairs whose id lies outside [0, E) are left zero.  Every launch goes to
    torch's current stream, so a step can be captured in a graph."""

    def __init__(self, codes, absmax, max_experts=None, wbuf=None):
        self.codes, self.absmax = codes, absmax
        E, N, half = codes.shape
        self.E, self.N, self.K = E, N, half * 2
        if wbuf is None:
            wbuf = torch.empty((max_experts or E, N, self.K), dtype=torch.bfloat16,
                               device=codes.device)
        if wbuf.dtype != torch.bfloat16 or tuple(wbuf.shape[1:]) != (N, self.K):
            raise ValueError("wbuf must be bf16 [max_experts, N, K]")
        self.wbuf = wbuf

    def plan(self, ids, gather):
        ids = np.asarray(ids, dtype=np.int64)
        rows, topk = ids.shape
        flat = ids.reshape(-1)
        experts = [int(e) for e in np.unique(flat) if 0 <= e < self.E]
        if len(experts) > self.wbuf.shape[0]:
            raise ValueError("more distinct experts than the bf16 buffer holds")
        dev = self.codes.device
        groups = []
        for j, e in enumerate(experts):
            pairs = np.flatnonzero(flat == e)
            src = pairs // topk if gather else pairs
            groups.append((j, e, torch.from_numpy(pairs).to(dev),
                           torch.from_numpy(src).to(dev)))
        return groups

    def decode(self, groups):
        if len(groups) == self.E and self.wbuf.shape[0] >= self.E:
            # every expert active (prefill): one launch over the whole bank
            gq_nf4_decode(self.codes, self.absmax, out_f32=False, out_bf16=self.wbuf[:self.E])
            return
        for j, e, _, _ in groups:
            gq_nf4_decode(self.codes[e], self.absmax[e], out_f32=False, out_bf16=self.wbuf[j])

    def multiply(self, x, groups, out):
        out.zero_()
        for j, _, pairs, src in groups:
            xe = x.index_select(0, src)
            out.index_copy_(0, pairs, torch.mm(xe, self.wbuf[j].t()))
        return out

    def run(self, x, groups, out):
        self.decode(groups)
        return self.multiply(x, groups, out)
