"""OCP e4m3 element format and the two-term activation split (test
infrastructure only).

The pages feed MXFP4 expert weights to the matmul as they are stored:
"Receipts-driven engineering", opening summary (MXFP4 as OCP e2m1 on a
checkpoint's released bytes) and the MXFP4 inference record ("How do I run
MoE expert inference natively on MXFP4 (e2m1 + e8m0) weights ...",
summary).  A block-scaled fp4 matrix instruction takes its other operand in
an MX format too (8-, 6- or 4-bit elements with an e8m0 scale per 32), while
the pages keep the activations in bf16 (weights-only 4-bit).  The reading
taken for that path: every bf16 activation is written as the sum of two
e4m3 terms, x ~= hi * 2^Xh + lo * 2^Xl, each term with its own e8m0 scale
per 32 consecutive activations of a row, the second term carrying the
rounding residual of the first.  The product then stays within the same
tolerance as the bf16 path (the split is close to bf16 precision), while
the matmul runs on the MX instruction.

Definitions (all exact; float64 on the host):

* e4m3 (OCP Microscaling Formats v1.0, FP8 E4M3): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 is subnormal
  (m/8 * 2^-6); S.1111.111 is NaN; there is no infinity; the largest finite
  magnitude is 448.
* ``e4m3_rne(v)``: the e4m3 code nearest to v (|v| <= 448), an exact tie
  going to the code with an even mantissa; the sign bit is the sign of v
  (a negative value that rounds to zero gives -0, code 0x80).
* block scale: for a block of 32 values with largest magnitude a > 0,
  X = the smallest integer with a * 2^-X <= 448 (= ceil(log2(a / 448))),
  clamped to [-127, 127]; X = -127 for an all-zero block.  The e8m0 byte
  is X + 127.
* split of one block: hi = e4m3_rne(x * 2^-Xh) with Xh from |x|; the
  residual r = x - e4m3(hi) * 2^Xh (exact); lo = e4m3_rne(r * 2^-Xl) with
  Xl from |r|.
"""

import math

import numpy as np

from .bf16 import bf16_to_f32

__all__ = ["E4M3_VALUES", "e4m3_value", "e4m3_rne", "block_scale_exponent", "act_split_e4m3",
           "act_split_value", "SPLIT_BLOCK"]

SPLIT_BLOCK = 32
E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of an 8-bit e4m3 code from its bit fields (NaN for S.1111.111)."""
    code = int(code)
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = math.ldexp(man / 8.0, -6)                   # subnormal
    else:
        mag = math.ldexp(1.0 + man / 8.0, exp - 7)
    return sign * mag


E4M3_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E4M3_VALUES.setflags(write=False)
_MAGS = E4M3_VALUES[:0x7F]                                # codes 0x00 .. 0x7E, ascending


def e4m3_rne(v):
    """float64 array (|v| <= 448, finite) -> uint8 e4m3 codes, nearest value,
    ties to the even mantissa, sign from the sign bit of v."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("e4m3_rne: values must be finite with magnitude <= 448")
    a = np.abs(v)
    hi = np.searchsorted(_MAGS, a, side="left")           # first magnitude >= a
    hi = np.minimum(hi, len(_MAGS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _MAGS[hi] - a
    d_lo = a - _MAGS[lo]
    exact = _MAGS[hi] == a
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    mag = np.where(exact, hi, np.where(pick_lo, lo, hi)).astype(np.uint8)
    return (mag | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def block_scale_exponent(amax):
    """X = smallest integer with amax * 2^-X <= 448, clamped to [-127, 127];
    -127 for amax == 0.  ``amax`` >= 0, float64 array."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    for idx in np.ndindex(amax.shape):
        a = float(amax[idx])
        if a == 0.0:
            continue
        f, e = math.frexp(a)                              # a = f * 2^e, f in [0.5, 1)
        X = e - 9                                         # a * 2^-X = f * 512 in [256, 512)
        if math.ldexp(a, -X) > E4M3_MAX:
            X += 1
        out[idx] = min(max(X, -127), 127)
    return out


def _split_term(v):
    """One term of the split over blocks: v float64 [..., nb, 32] ->
    (codes uint8 [..., nb, 32], X int [..., nb], value float64 [..., nb, 32])."""
    X = block_scale_exponent(np.abs(v).max(axis=-1))
    scaled = np.ldexp(v, -X[..., None])
    codes = e4m3_rne(scaled)
    value = np.ldexp(E4M3_VALUES[codes], X[..., None])
    return codes, X, value


def act_split_e4m3(x_bits):
    """Two-term e4m3 split of bf16 activations.

    x_bits  uint16 bf16 [rows, K], K a multiple of 32
    returns (hi uint8 [rows, K], lo uint8 [rows, K],
             s_hi uint8 [rows, K/32], s_lo uint8 [rows, K/32])  (e8m0 bytes)
    """
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    rows, K = x.shape
    if K % SPLIT_BLOCK:
        raise ValueError("K must be a multiple of 32")
    xb = x.reshape(rows, K // SPLIT_BLOCK, SPLIT_BLOCK)
    hi, Xh, hv = _split_term(xb)
    r = xb - hv                                           # exact residual
    lo, Xl, _ = _split_term(r)
    return (hi.reshape(rows, K), lo.reshape(rows, K), (Xh + 127).astype(np.uint8),
            (Xl + 127).astype(np.uint8))


def act_split_value(hi, lo, s_hi, s_lo):
    """The activations the split represents: hi * 2^(s_hi-127) +
    lo * 2^(s_lo-127), float64 [rows, K]."""
    rows, K = hi.shape
    nb = K // SPLIT_BLOCK
    Xh = s_hi.astype(np.int64) - 127
    Xl = s_lo.astype(np.int64) - 127
    v = (np.ldexp(E4M3_VALUES[hi].reshape(rows, nb, SPLIT_BLOCK), Xh[..., None])
         + np.ldexp(E4M3_VALUES[lo].reshape(rows, nb, SPLIT_BLOCK), Xl[..., None]))
    return v.reshape(rows, K)
