"""Grouped expert matmul and its input gradient, in float64 (test
infrastructure only).

What is computed ("grouped-nf4-gemm 0.43.0", section "Which entry
point?": grouped NF4 forward and backward, native MXFP4 expert math;
"Receipts-driven engineering", opening summary: the experts' matmuls run
directly on 4-bit packed weights and the NF4 path is differentiable;
"flashrt/grouped-moe-gemv", section "Functions": one product per routed
slot, ``[M, top_k]`` routing, ``[M, top_k, N]`` output, and for
projections whose input differs per routed pair the caller flattens to
``M = pairs, top_k = 1``):

* forward, for every pair ``p = t * top_k + s`` routed to a valid expert
  ``e = ids[t, s]``:  ``Y[p, n] = sum_k X[t, k] * W_e[n, k]``;
* input gradient, for every pair ``p`` with expert ``e(p)``:
  ``dX[p, k] = sum_n dY[p, n] * W_e(p)[n, k]``.

Readings taken where the pages are silent:

* Activations are the exact bf16 values given (weights-only 4-bit, W4A16);
  weights are the exact decoded float32 values; the sum is evaluated in
  float64 (a library matmul in float64 is used as the summation step).
* An optional per-pair scale (router weight) multiplies the pair's output.
* A pair whose expert id is outside ``[0, E)`` is dropped: its output row
  is zero.
* A GPU result is accepted when, for every expert with at least one
  pair, the relative L2 error of that expert's output rows is at most
  4e-3 (and rows whose reference is exactly zero are exactly zero).
"""

import numpy as np

from .bf16 import bf16_to_f32

__all__ = ["grouped_gemm", "grouped_dgrad", "brute_force_gemm", "brute_force_dgrad",
           "compare_slices", "REL_L2_TOL"]

REL_L2_TOL = 4e-3


def _weights_of(weights, e):
    """``weights`` is a [E, N, K] float32 array or a callable e -> [N, K]."""
    w = weights(e) if callable(weights) else weights[e]
    return np.asarray(w, dtype=np.float32).astype(np.float64)


def grouped_gemm(x_bits, weights, topk_ids, num_experts, pair_scale=None):
    """Forward grouped product.

    x_bits     uint16 bf16 [rows, K]
    weights    float32 [E, N, K] or callable e -> float32 [N, K]
    topk_ids   int [rows, top_k]
    returns    float64 [rows * top_k, N]
    """
    x = bf16_to_f32(x_bits).astype(np.float64)
    ids = np.asarray(topk_ids).astype(np.int64)
    rows, topk = ids.shape
    flat = ids.reshape(-1)
    P = rows * topk
    N = None
    out = None
    for e in range(num_experts):
        pairs = np.nonzero(flat == e)[0]
        if len(pairs) == 0:
            continue
        w = _weights_of(weights, e)                       # [N, K] float64
        if out is None:
            N = w.shape[0]
            out = np.zeros((P, N), dtype=np.float64)
        out[pairs] = x[pairs // topk] @ w.T
    if out is None:
        w0 = _weights_of(weights, 0)
        out = np.zeros((P, w0.shape[0]), dtype=np.float64)
    if pair_scale is not None:
        out *= np.asarray(pair_scale, dtype=np.float32).reshape(-1).astype(np.float64)[:, None]
    return out


def grouped_dgrad(dy_bits, weights, pair_expert, num_experts):
    """Input gradient through the frozen experts.

    dy_bits      uint16 bf16 [P, N]
    weights      float32 [E, N, K] or callable e -> float32 [N, K]
    pair_expert  int [P]
    returns      float64 [P, K]
    """
    dy = bf16_to_f32(dy_bits).astype(np.float64)
    pe = np.asarray(pair_expert).reshape(-1).astype(np.int64)
    P = dy.shape[0]
    out = None
    for e in range(num_experts):
        pairs = np.nonzero(pe == e)[0]
        if len(pairs) == 0:
            continue
        w = _weights_of(weights, e)
        if out is None:
            out = np.zeros((P, w.shape[1]), dtype=np.float64)
        out[pairs] = dy[pairs] @ w
    if out is None:
        w0 = _weights_of(weights, 0)
        out = np.zeros((P, w0.shape[1]), dtype=np.float64)
    return out


def brute_force_gemm(x_bits, weights, topk_ids, num_experts, pair_scale=None):
    """Same result as ``grouped_gemm`` from plain per-token, per-slot,
    per-output loops (tiny inputs only)."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    ids = np.asarray(topk_ids).astype(np.int64)
    rows, topk = ids.shape
    w_all = [_weights_of(weights, e) for e in range(num_experts)]
    N, K = w_all[0].shape
    out = np.zeros((rows * topk, N), dtype=np.float64)
    for t in range(rows):
        for s in range(topk):
            e = int(ids[t, s])
            if not 0 <= e < num_experts:
                continue
            p = t * topk + s
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += x[t, k] * w_all[e][n, k]
                if pair_scale is not None:
                    acc *= float(np.float32(np.asarray(pair_scale).reshape(-1)[p]))
                out[p, n] = acc
    return out


def brute_force_dgrad(dy_bits, weights, pair_expert, num_experts):
    """Same result as ``grouped_dgrad`` from plain loops (tiny inputs only)."""
    dy = bf16_to_f32(dy_bits).astype(np.float64)
    pe = np.asarray(pair_expert).reshape(-1).astype(np.int64)
    w_all = [_weights_of(weights, e) for e in range(num_experts)]
    N, K = w_all[0].shape
    out = np.zeros((dy.shape[0], K), dtype=np.float64)
    for p in range(dy.shape[0]):
        e = int(pe[p])
        if not 0 <= e < num_experts:
            continue
        for k in range(K):
            acc = 0.0
            for n in range(N):
                acc += dy[p, n] * w_all[e][n, k]
            out[p, k] = acc
    return out


def compare_slices(y_test, y_ref, pair_expert, num_experts, tol=REL_L2_TOL):
    """Per-expert relative L2 error of ``y_test`` against the float64 reference.

    Returns (ok, errors) where ``errors[e]`` is the relative error over the
    rows of expert ``e`` (``None`` for experts without pairs).  Rows of
    dropped pairs (expert id outside [0, E)), and the rows of an expert
    whose reference is exactly zero, must be exactly zero in ``y_test``.
    """
    yt = np.asarray(y_test, dtype=np.float64)
    yr = np.asarray(y_ref, dtype=np.float64)
    pe = np.asarray(pair_expert).reshape(-1).astype(np.int64)
    if yt.shape != yr.shape:
        return False, {"shape": (yt.shape, yr.shape)}
    if not np.all(np.isfinite(yt)):
        return False, {"nonfinite": int(np.sum(~np.isfinite(yt)))}
    errors = {}
    ok = True
    for e in range(num_experts):
        rows = np.nonzero(pe == e)[0]
        if len(rows) == 0:
            errors[e] = None
            continue
        ref = yr[rows]
        nrm = np.linalg.norm(ref)
        if nrm == 0:
            err = 0.0 if np.all(yt[rows] == 0) else np.inf
        else:
            err = float(np.linalg.norm(yt[rows] - ref) / nrm)
        errors[e] = err
        if not err <= tol:
            ok = False
    dropped = np.nonzero((pe < 0) | (pe >= num_experts))[0]
    if len(dropped) and not np.all(yt[dropped] == 0):
        ok = False
        errors["dropped"] = "nonzero"
    return ok, errors
