"""The mixture-of-experts layer around the grouped products, in float64
(test infrastructure only).

The pages describe the expert matmuls of a mixture-of-experts block
("grouped-nf4-gemm 0.43.0", page header: the active experts' products in
one launch; section "Which entry point?": the grouped NF4 forward and the
per-slot routing) and benchmark them on the Qwen3-30B-A3B expert shapes,
whose experts are gated-linear-unit MLPs: a gate and an up projection of
the hidden vector, their SwiGLU product, then the down projection; a
token's output is the router-weighted sum of its top_k experts' outputs
("flashrt/grouped-moe-gemv", section "Functions": [M, top_k] routing and
[M, top_k, N] per-slot outputs, which the caller reduces over top_k).

Readings taken where the pages are silent:

* a fused gate_up weight [2I, H] holds the gate projection in rows
  [0, I) and the up projection in rows [I, 2I);
* the activation is SwiGLU, act = silu(gate) * up with
  silu(z) = z / (1 + exp(-z)), applied to the exact products;
* the combine is the router-weighted sum over a token's slots; weights
  None means an unweighted sum (the router weight was already applied per
  pair).

The pages also run gpt-oss's MXFP4 experts ("Receipts-driven engineering",
"The numbers": the gpt-oss-120b MXFP4 serving row; the MXFP4 inference
record, summary) without defining that model's expert activation.  Reading
taken: gpt-oss's published expert MLP, whose fused gate_up weight
interleaves the two projections (row 2j: gate j, row 2j + 1: up j) and whose
activation clamps both and shifts the linear term,

    act(g, u) = gc * sigmoid(alpha * gc) * (uc + 1),
    gc = min(g, limit),  uc = min(max(u, -limit), limit),

with alpha = 1.702 and limit = 7 (``swiglu_oss``).  The model's projection
biases are not part of the products the pages define and are left out.
"""

import numpy as np

from .bf16 import bf16_to_f32
from .grouped import grouped_gemm

__all__ = ["silu", "swiglu", "gate_up_swiglu", "combine", "down_combine", "OSS_ALPHA",
           "OSS_LIMIT", "swiglu_oss", "gate_up_swiglu_oss"]

OSS_ALPHA = 1.702
OSS_LIMIT = 7.0


def silu(z):
    """z * sigmoid(z), elementwise, float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def swiglu(h):
    """[P, 2I] gate_up products -> [P, I] activations (gate rows first)."""
    h = np.asarray(h, dtype=np.float64)
    two_i = h.shape[1]
    if two_i % 2:
        raise ValueError("gate_up width must be even")
    i = two_i // 2
    return silu(h[:, :i]) * h[:, i:]


def swiglu_oss(h, alpha=OSS_ALPHA, limit=OSS_LIMIT):
    """[P, 2I] gate_up products, gate and up interleaved (columns 2j, 2j+1)
    -> [P, I]: the clamped, shifted gated unit of the module docstring."""
    h = np.asarray(h, dtype=np.float64)
    if h.shape[1] % 2:
        raise ValueError("gate_up width must be even")
    gate = np.minimum(h[:, 0::2], limit)
    up = np.clip(h[:, 1::2], -limit, limit)
    return gate / (1.0 + np.exp(-alpha * gate)) * (up + 1.0)


def gate_up_swiglu_oss(x_bits, weights, topk_ids, num_experts, alpha=OSS_ALPHA,
                       limit=OSS_LIMIT):
    """gpt-oss activation of every routed pair's gate_up product: float64 [P, I]."""
    return swiglu_oss(grouped_gemm(x_bits, weights, topk_ids, num_experts), alpha, limit)


def gate_up_swiglu(x_bits, weights, topk_ids, num_experts):
    """SwiGLU of every routed pair's gate_up product: float64 [P, I]."""
    return swiglu(grouped_gemm(x_bits, weights, topk_ids, num_experts))


def combine(y_pairs, topk, weights=None):
    """Per-token sum over its top_k slots: [rows*topk, H] -> [rows, H].

    weights: float32 [rows, topk] router weights, or None (plain sum)."""
    y = np.asarray(y_pairs, dtype=np.float64)
    P, H = y.shape
    if P % topk:
        raise ValueError("rows * topk pairs expected")
    y = y.reshape(P // topk, topk, H)
    if weights is not None:
        w = np.asarray(weights, dtype=np.float32).astype(np.float64).reshape(P // topk, topk)
        y = y * w[:, :, None]
    return y.sum(axis=1)


def down_combine(act_bits, weights, topk_ids, num_experts, topk_weights=None):
    """Down projection of every pair's activation row, then the combine.

    act_bits      uint16 bf16 [rows*topk, I] (row p is pair p's input)
    weights       float32 [E, H, I] or callable e -> [H, I]
    topk_ids      int [rows, topk]
    topk_weights  float32 [rows, topk] or None
    returns       float64 [rows, H]
    """
    ids = np.asarray(topk_ids)
    y = grouped_gemm(act_bits, weights, ids.reshape(-1, 1), num_experts)
    return combine(y, ids.shape[1], topk_weights)
