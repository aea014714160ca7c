"""Pins for the oracle's e4m3 format and two-term activation split.

* e4m3 values against facts of the OCP MX v1.0 FP8 E4M3 encoding
  (hand-written in tests/golden/pages_examples.json);
* e4m3 rounding against a brute-force nearest search over every code, with
  planted ties;
* the block scale rule as an inequality (smallest X with amax * 2^-X <= 448);
* the split is exact on blocks whose magnitudes span less than 2^12 (a
  bf16 value has 8 significant bits: the first term holds the top 4, the
  residual the rest), and within 2^-8 |x| + 2^-16 amax everywhere (two
  rounding steps of at most 2^-4 relative each).
"""

import math

import numpy as np
import pytest

import oracle
from oracle.fp8 import (E4M3_VALUES, act_split_e4m3, act_split_value, block_scale_exponent,
                        e4m3_rne)


def test_e4m3_facts(golden):
    facts = golden["e4m3_facts"]
    for code, val in facts["codes"].items():
        got = E4M3_VALUES[int(code, 16)]
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in facts["nan_codes"]:
        assert math.isnan(E4M3_VALUES[int(code, 16)])
    mags = E4M3_VALUES[:128]
    finite = mags[np.isfinite(mags)]
    assert len(finite) == facts["finite_magnitudes"]
    assert np.all(np.diff(finite) > 0)                     # ascending, distinct
    assert np.array_equal(E4M3_VALUES[128:][np.isfinite(E4M3_VALUES[128:])], -finite)


def _nearest_brute(v):
    best, bd = None, None
    for c in range(0x7F):                                  # finite magnitudes
        d = abs(abs(v) - E4M3_VALUES[c])
        if bd is None or d < bd or (d == bd and c % 2 == 0 and best % 2 == 1):
            best, bd = c, d
    return best | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_rne_against_brute_force():
    g = np.random.default_rng(1)
    v = np.concatenate([g.uniform(-448, 448, 400), g.normal(0, 1, 400),
                        g.normal(0, 1e-2, 200) * 2.0 ** g.integers(-8, 0, 200),
                        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, -(2.0 ** -11)]])
    got = e4m3_rne(v)
    want = np.array([_nearest_brute(float(a)) for a in v], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_ties_go_to_even():
    mags = E4M3_VALUES[:0x7F]
    mid = (mags[:-1] + mags[1:]) / 2.0                     # exact midpoints
    got = e4m3_rne(mid)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    assert np.array_equal(e4m3_rne(-mid), (want | 0x80).astype(np.uint8))


def test_block_scale_rule():
    g = np.random.default_rng(2)
    a = np.concatenate([np.abs(g.normal(0, 1, 500)) * 2.0 ** g.integers(-40, 40, 500),
                        [448.0, 449.0, 1.0, 1.75, 1.7500001, 2.0 ** -20]])
    X = block_scale_exponent(a)
    for ai, xi in zip(a, X):
        assert math.ldexp(ai, -int(xi)) <= 448.0
        assert math.ldexp(ai, -(int(xi) - 1)) > 448.0      # X is the smallest such
    assert block_scale_exponent(np.array([0.0]))[0] == -127


def _blocks_within(g, rows, K, span_log2):
    """bf16 bit patterns whose magnitudes, per 32-block, lie within 2^span."""
    import torch
    e = g.integers(-20, 20, (rows, K // 32, 1))
    mag = 2.0 ** (e + g.uniform(0, span_log2, (rows, K // 32, 32)))
    x = (mag * g.choice([-1.0, 1.0], (rows, K // 32, 32))).reshape(rows, K).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_split_is_exact_on_narrow_blocks():
    g = np.random.default_rng(3)
    x = _blocks_within(g, 16, 256, 11.9)
    hi, lo, sh, sl = act_split_e4m3(x)
    back = act_split_value(hi, lo, sh, sl)
    assert np.array_equal(back, oracle.bf16_to_f32(x).astype(np.float64))


def test_split_error_bound_and_codes():
    import workloads as wl
    g = np.random.default_rng(4)
    x = wl.draw_bf16(g, (64, 2880))
    x[0, :32] = 0                                          # an all-zero block
    x[1, 32:64] = 0x8000                                   # -0 block
    hi, lo, sh, sl = act_split_e4m3(x)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    back = act_split_value(hi, lo, sh, sl)
    amax = np.abs(xf).reshape(64, -1, 32).max(axis=-1)
    bound = 2.0 ** -8 * np.abs(xf) + 2.0 ** -16 * np.repeat(amax, 32, axis=1)
    assert np.all(np.abs(back - xf) <= bound)
    assert sh[0, 0] == 0 and sl[0, 0] == 0 and not hi[0, :32].any() and not lo[0, :32].any()
    rel = np.linalg.norm(back - xf) / np.linalg.norm(xf)
    assert rel < 2.0 ** -8
    # every code is finite and scaled values stayed within range
    assert np.all(np.isfinite(E4M3_VALUES[hi])) and np.all(np.isfinite(E4M3_VALUES[lo]))


def test_split_planted_mistake_is_caught():
    """Dropping the second term breaks the bound (the pin is not vacuous)."""
    import workloads as wl
    x = wl.draw_bf16(np.random.default_rng(5), (8, 256))
    hi, lo, sh, sl = act_split_e4m3(x)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    one_term = act_split_value(hi, np.zeros_like(lo), sh, sl)
    amax = np.abs(xf).reshape(8, -1, 32).max(axis=-1)
    bound = 2.0 ** -8 * np.abs(xf) + 2.0 ** -16 * np.repeat(amax, 32, axis=1)
    assert np.any(np.abs(one_term - xf) > bound)


def test_e4m3_rne_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        e4m3_rne(np.array([np.nan]))
