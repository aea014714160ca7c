"""MXFP4 (e2m1 codes + e8m0 block scales) pack / decode for the oracle
(test infrastructure only).

What the pages fix ("grouped-nf4-gemm 0.43.0", section "Try the packers
and byte checks on CPU", MXFP4 round-trip example; "Receipts-driven
engineering", opening summary; the native-MXFP4 inference record's
summary):

* weights ``[..., K]`` with ``K % 32 == 0`` pack into ``uint8 [..., K/32, 16]``
  blocks (32 e2m1 codes per 16 bytes) plus ``uint8 [..., K/32]`` e8m0
  scales (printed example ``[128, 256] -> [128, 8, 16] + [128, 8]``);
* the element format is OCP e2m1; the round-trip relative error on
  standard-normal weights is about 0.12;
* the kernels consume a checkpoint's released bytes as they are.

Readings taken where the pages are silent (the OCP Microscaling
specification v1.0 supplies the format definitions):

* e2m1: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0;
  exponent 0 is subnormal (value = mantissa * 0.5).  Magnitudes are
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* e8m0 scale byte ``s`` means ``2**(s - 127)``; 255 is NaN.
* Shared exponent of a block: ``X = floor(log2(amax)) - 2`` (2 is the
  largest e2m1 exponent), computed exactly with ``frexp``; clamped to
  [-127, 127]; an all-zero block uses X = -127.
* Element: ``v = w * 2**-X`` rounded to the nearest e2m1 magnitude, ties to
  the even mantissa, magnitudes above 6 saturate to 6; the sign bit is
  the sign bit of ``w`` (so a negative value that rounds to zero keeps
  code 8, -0).
* Nibble order: element ``2j`` in the LOW nibble of byte ``j`` (the layout
  of released gpt-oss checkpoints).
"""

import numpy as np

__all__ = ["E2M1_VALUES", "e2m1_value", "mxfp4_pack", "mxfp4_decode",
           "MX_BLOCK"]

MX_BLOCK = 32


def e2m1_value(code):
    """Value of a 4-bit e2m1 code from its bit fields (OCP MX v1.0)."""
    code = int(code)
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        mag = man * 0.5                                   # subnormal: 2**(1-1) * m/2
    else:
        mag = 2.0 ** (exp - 1) * (1.0 + man * 0.5)
    return sign * mag


E2M1_VALUES = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_VALUES.setflags(write=False)
_MAGS = E2M1_VALUES[:8]                                   # 0, .5, 1, 1.5, 2, 3, 4, 6


def _round_e2m1_magnitude(v):
    """Index 0..7 of the e2m1 magnitude nearest to ``v >= 0`` (float64),
    ties to the even index (mantissa bit 0), saturating above 6."""
    v = np.minimum(v, 6.0)
    d = np.abs(v[..., None] - _MAGS)                      # [..., 8]
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                      # one or two candidates
    idx = np.arange(8)
    # among the nearest candidates prefer an even index, else the lowest
    even_pick = np.where(cand & (idx % 2 == 0), idx, 99).min(axis=-1)
    any_pick = np.where(cand, idx, 99).min(axis=-1)
    return np.where(even_pick < 99, even_pick, any_pick).astype(np.uint8)


def mxfp4_pack(w):
    """Quantise float32 ``w [..., K]`` -> (blocks uint8 [..., K/32, 16], scales uint8 [..., K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.shape[-1] % MX_BLOCK:
        raise ValueError("K must be a multiple of 32 for MXFP4")
    lead = w.shape[:-1]
    nb = w.shape[-1] // MX_BLOCK
    blk = w.reshape(lead + (nb, MX_BLOCK)).astype(np.float64)
    amax = np.abs(blk).max(axis=-1)                                   # [..., nb]
    _, ex = np.frexp(amax)                 # amax = f * 2**ex, f in [0.5, 1)
    x = ex.astype(np.int64) - 1 - 2        # floor(log2 amax) - emax(e2m1)
    x = np.where(amax == 0, -127, x)
    x = np.clip(x, -127, 127)
    scaled = np.abs(blk) * np.ldexp(1.0, -x)[..., None]               # exact power-of-2 scaling
    mag = _round_e2m1_magnitude(scaled)
    sign = np.signbit(blk.astype(np.float32)).astype(np.uint8)
    codes = (sign << 3) | mag                                         # [..., nb, 32]
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    scales = (x + 127).astype(np.uint8)
    return packed, scales


def mxfp4_decode(blocks, scales):
    """Decode (blocks uint8 [..., K/32, 16], scales uint8 [..., K/32]) -> float32 [..., K].

    Each weight is ``e2m1(code) * 2**(s - 127)`` evaluated exactly in float64
    and stored as float32 (exact for every finite case; overflow gives inf);
    scale byte 255 decodes to NaN.
    """
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    if blocks.shape[-1] != 16 or blocks.shape[:-1] != scales.shape:
        raise ValueError("blocks must be [..., K/32, 16] and scales [..., K/32]")
    codes = np.empty(blocks.shape[:-1] + (32,), dtype=np.uint8)
    codes[..., 0::2] = blocks & 0x0F        # element 2j: low nibble
    codes[..., 1::2] = blocks >> 4          # element 2j+1: high nibble
    vals = E2M1_VALUES[codes]                                          # float64
    s = scales.astype(np.int64)
    factor = np.ldexp(1.0, s - 127)
    out = vals * factor[..., None]
    out = np.where((s == 255)[..., None], np.nan, out)
    with np.errstate(over="ignore"):
        out32 = out.astype(np.float32)
    return out32.reshape(blocks.shape[:-2] + (blocks.shape[-2] * 32,))

