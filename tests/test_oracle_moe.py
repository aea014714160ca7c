"""Pins of the MoE-layer oracle (oracle/moe.py) against closed forms,
brute force and layout probes."""

import math

import numpy as np
import pytest

import oracle
import workloads as wl


def test_silu_closed_forms():
    # sigmoid(1) = e / (1 + e); silu(-z) = silu(z) - z
    s1 = math.e / (1.0 + math.e)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1.0) == pytest.approx(s1, rel=1e-15)
    assert oracle.silu(-1.0) == pytest.approx(s1 - 1.0, rel=1e-14)
    z = np.linspace(-9, 9, 37)
    np.testing.assert_allclose(oracle.silu(-z), oracle.silu(z) - z, rtol=0, atol=1e-14)
    # large |z|: identity and (almost) zero
    assert oracle.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_swiglu_brute_force():
    g = np.random.default_rng(0)
    h = g.standard_normal((5, 6)) * 3
    want = np.array([[h[p, j] / (1 + math.exp(-h[p, j])) * h[p, 3 + j] for j in range(3)]
                     for p in range(5)])
    np.testing.assert_allclose(oracle.swiglu(h), want, rtol=1e-14, atol=0)
    with pytest.raises(ValueError):
        oracle.swiglu(np.zeros((2, 5)))


def test_gate_rows_come_first():
    """Zero gate rows give silu(0) * up = 0 everywhere; up rows that select
    x[:, 0] give silu(gate) * x[:, 0], checked against the gate product
    computed directly.  A layout with the up rows first fails both."""
    g = np.random.default_rng(1)
    E, I, H = 2, 4, 64
    x = wl.draw_bf16(g, (3, H))
    ids = np.array([[0, 1], [1, 0], [1, 1]])
    W = g.standard_normal((E, 2 * I, H)).astype(np.float32)
    W_gate0 = W.copy()
    W_gate0[:, :I] = 0
    assert not oracle.gate_up_swiglu(x, W_gate0, ids, E).any()
    W_up_const = W.copy()
    W_up_const[:, I:] = 0
    W_up_const[:, I:, 0] = 1.0                     # up = x[:, 0] for every j
    act = oracle.gate_up_swiglu(x, W_up_const, ids, E)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    gate = np.stack([xf[p // 2] @ W[ids.reshape(-1)[p], :I].astype(np.float64).T
                     for p in range(6)])
    want = gate / (1 + np.exp(-gate)) * xf[np.arange(6) // 2, :1]
    np.testing.assert_allclose(act, want, rtol=1e-12, atol=1e-12)


def test_combine_one_hot_and_uniform():
    g = np.random.default_rng(2)
    rows, topk, H = 4, 3, 7
    y = g.standard_normal((rows * topk, H))
    w = np.zeros((rows, topk), np.float32)
    pick = np.array([2, 0, 1, 2])
    w[np.arange(rows), pick] = 1.0
    np.testing.assert_array_equal(oracle.combine(y, topk, w), y[np.arange(rows) * topk + pick])
    same = np.repeat(g.standard_normal((rows, 1, H)), topk, axis=1).reshape(rows * topk, H)
    u = np.full((rows, topk), 0.25, np.float32)
    np.testing.assert_allclose(oracle.combine(same, topk, u), same[::topk] * 0.75, rtol=1e-15)
    np.testing.assert_allclose(oracle.combine(y, topk), y.reshape(rows, topk, H).sum(1))


def test_down_combine_brute_force():
    g = np.random.default_rng(3)
    E, I, H, rows, topk = 3, 64, 5, 2, 2
    act = wl.draw_bf16(g, (rows * topk, I))
    W = g.standard_normal((E, H, I)).astype(np.float32)
    ids = np.array([[2, 0], [1, 2]])
    w = np.array([[0.75, 0.25], [0.5, 0.5]], np.float32)
    af = oracle.bf16_to_f32(act).astype(np.float64)
    want = np.zeros((rows, H))
    for t in range(rows):
        for s in range(topk):
            p = t * topk + s
            for n in range(H):
                want[t, n] += float(w[t, s]) * sum(af[p, i] * float(W[ids[t, s], n, i])
                                                   for i in range(I))
    np.testing.assert_allclose(oracle.down_combine(act, W, ids, E, w), want, rtol=1e-12,
                               atol=1e-12)


# ---- gpt-oss activation (interleaved gate/up, clamped, shifted) ----

def _oss(g, u, **kw):
    """act(g, u) through the oracle's [P, 2I] interface (one pair per row)."""
    g, u = np.broadcast_arrays(np.asarray(g, np.float64), np.asarray(u, np.float64))
    h = np.stack([g.ravel(), u.ravel()], axis=1)
    return oracle.swiglu_oss(h, **kw).ravel().reshape(g.shape)


def test_oss_gate_odd_part():
    """sigmoid(t) + sigmoid(-t) = 1 makes act(g, u) - act(-g, u) = g (u + 1)
    for |g| <= limit (a flipped sign, a dropped shift or alpha applied
    outside the sigmoid breaks it)."""
    g = np.linspace(-6.9, 6.9, 47)[:, None]
    u = np.linspace(-6.5, 6.5, 11)[None, :]
    np.testing.assert_allclose(_oss(g, u) - _oss(-g, u), g * (u + 1.0), rtol=0, atol=1e-13)


def test_oss_zeros_and_shift():
    u = np.linspace(-10, 10, 21)
    assert not _oss(0.0, u).any()                          # gated part vanishes at g = 0
    g = np.linspace(-9, 9, 19)
    assert not _oss(g, -1.0).any()                         # the +1 shift cancels u = -1


def test_oss_clamps():
    g = np.linspace(-3, 3, 13)
    np.testing.assert_array_equal(_oss(g, 50.0), _oss(g, 7.0))       # up clamped above
    np.testing.assert_array_equal(_oss(g, -50.0), _oss(g, -7.0))     # and below
    u = np.linspace(-3, 3, 13)
    np.testing.assert_array_equal(_oss(100.0, u), _oss(7.0, u))      # gate clamped above only
    # no lower clamp on the gate: a very negative gate drives the unit to 0
    # from below, unlike a clamp at -7 (which would give about -7e-6 * (u+1))
    assert np.all(np.abs(_oss(-30.0, u)) < 1e-20)
    assert np.all(np.abs(_oss(-7.0, u + 4.0)) > 1e-6)


def test_oss_alpha_against_silu():
    """g * sigmoid(alpha g) = silu(alpha g) / alpha, checked against the
    pinned silu at alpha = 1 and 2 with no clamping in reach."""
    g = np.linspace(-5, 5, 41)[:, None]
    u = np.array([[-0.5, 0.0, 2.0]])
    for a in (1.0, 2.0):
        want = oracle.silu(a * g) / a * (u + 1.0)
        np.testing.assert_allclose(_oss(g, u, alpha=a, limit=1e9), want, rtol=1e-14, atol=1e-15)
    # slope of the gated part at 0 is sigmoid(0) = 1/2, whatever alpha
    eps = 1e-6
    slope = (_oss(eps, 0.0) - _oss(-eps, 0.0)) / (2 * eps)
    assert slope == pytest.approx(0.5, rel=1e-9)


def test_oss_interleaved_layout():
    """Gate rows are the even rows of the fused weight: zero even rows give
    act = 0; zero odd rows give act = gate * sigmoid(alpha gate) exactly as
    computed from the even-row product.  The split-halves layout fails both."""
    g = np.random.default_rng(4)
    E, I, H = 2, 4, 64
    x = wl.draw_bf16(g, (3, H))
    ids = np.array([[0, 1], [1, 0], [1, 1]])
    W = (g.standard_normal((E, 2 * I, H)) * 0.2).astype(np.float32)
    W_gate0 = W.copy()
    W_gate0[:, 0::2] = 0
    assert not oracle.gate_up_swiglu_oss(x, W_gate0, ids, E).any()
    W_up0 = W.copy()
    W_up0[:, 1::2] = 0
    act = oracle.gate_up_swiglu_oss(x, W_up0, ids, E)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    gate = np.stack([xf[p // 2] @ W[ids.reshape(-1)[p], 0::2].astype(np.float64).T
                     for p in range(6)])
    assert np.abs(gate).max() < 7.0                        # no clamping in reach
    np.testing.assert_allclose(act, oracle.silu(oracle.OSS_ALPHA * gate) / oracle.OSS_ALPHA,
                               rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.swiglu_oss(np.zeros((2, 5)))
