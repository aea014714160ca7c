"""bfloat16 rounding used by the oracle (test infrastructure only).

The pages name bf16 as the dense type the method avoids materialising
("Receipts-driven engineering", opening summary: no dequantize-to-bf16
round trip) and as the activation / output type of the grouped API
("flashrt/grouped-moe-gemv", section "Functions": BF16 activations,
BF16 outputs).  They do not state a rounding mode; the reading taken is
IEEE round-to-nearest, ties-to-even (RNE), which is the usual definition.

The conversion below is written from that definition -- pick the nearer of
the two bf16 neighbours, ties to the even significand -- rather than with
the well-known integer-add trick, so that a reader can check it by eye.
"""

import numpy as np

__all__ = ["f32_to_bf16_rne", "bf16_to_f32", "bf16_bits_value_f64"]


def bf16_bits_value_f64(bits):
    """Exact value of bf16 bit patterns as float64, treating the all-ones
    exponent as an ordinary (unbounded) exponent.  Used only to measure
    distances to rounding candidates; callers handle inf / NaN inputs
    separately."""
    b = np.asarray(bits, dtype=np.uint32)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    exp = ((b >> 7) & 0xFF).astype(np.int64)
    man = (b & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + man / 128.0, (exp - 127).astype(np.int64))
    sub = sign * np.ldexp(man / 128.0, -126)
    return np.where(exp == 0, sub, normal)


def f32_to_bf16_rne(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.

    For a finite input the two candidates are the bf16 values adjacent to
    it in magnitude: ``lo`` (truncate toward zero) and ``hi`` (the next
    bf16 away from zero).  The nearer one wins; an exact tie goes to the
    candidate whose last significand bit is 0.  A value at or past the
    midpoint between the largest finite bf16 and 2**128 becomes infinity,
    which falls out of treating the all-ones exponent as unbounded.
    Infinities keep their sign; every NaN becomes the quiet NaN 0x7FC0 with
    the input's sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lo = (u >> 16).astype(np.uint32)            # truncation toward zero
    hi = lo + 1                                  # next bf16 away from zero
    xv = x.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        d_lo = np.abs(xv - bf16_bits_value_f64(lo))
        d_hi = np.abs(bf16_bits_value_f64(hi) - xv)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    out = np.where(take_hi, hi, lo).astype(np.uint32)
    exact = (u & 0xFFFF) == 0                    # already representable
    out = np.where(exact, lo, out)
    is_inf = np.isinf(x)
    out = np.where(is_inf, lo, out)              # lo is the exact inf pattern
    is_nan = np.isnan(x)
    out = np.where(is_nan, (u >> 16) & 0x8000 | 0x7FC0, out)
    return out.astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 (exact: bf16 is the top half of
    an IEEE binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
