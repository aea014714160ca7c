"""NF4 pack / decode for the oracle (test infrastructure only).

What the pages fix ("grouped-nf4-gemm 0.43.0", section "Try the packers
and byte checks on CPU", NF4 round-trip example, and "Receipts-driven
engineering", opening summary):

* an expert weight is ``[N, K]``; packing yields ``uint8 [N, K/2]`` codes
  (two 4-bit codes per byte) and ``float32 [N, K/64]`` absmax, i.e. one
  absmax per 64-element block along K (the printed example is
  ``[256, 512] -> [256, 256] u8 + [256, 8] fp32``);
* the codes index a 16-entry normal-float codebook, the bitsandbytes
  packed format unchanged;
* round-trip relative error on standard-normal weights is about 0.09 and
  re-packing the decoded weights reproduces the packed bytes.

Readings taken where the pages are silent:

* Codebook values: the NF4 data type published with QLoRA (Dettmers et
  al., 2023), written below as float32 bit patterns.  The CPU tests
  rebuild it from its normal-quantile definition as an independent check.
* Nibble order: element ``2j`` of a row sits in the HIGH nibble of byte
  ``j``, element ``2j+1`` in the low nibble (the bitsandbytes convention
  the pages say is kept unchanged).
* Normalisation: ``y = float32(w / absmax)`` with ``absmax`` the float32
  maximum magnitude of the block; an all-zero block stores absmax 0 and
  code 7 (the 0.0 entry) everywhere.
* Code choice: the nearest codebook entry to ``y``; an exact tie goes to
  the lower index.
* Decode: ``w = float32(q[code] * absmax)``, one IEEE float32 multiply
  rounded to nearest even.
"""

import numpy as np

__all__ = ["NF4_CODEBOOK", "NF4_BLOCK", "nf4_pack", "nf4_decode"]

NF4_BLOCK = 64

# NF4 codebook (QLoRA, Dettmers et al. 2023), index -> float32 bit pattern.
_NF4_BITS = [
    0xBF800000,  # -1.0
    0xBF3239B1,  # -0.6961928009986877
    0xBF066B30,  # -0.5250730514526367
    0xBECA32A0,  # -0.39491748809814453
    0xBE91A24D,  # -0.28444138169288635
    0xBE3D353F,  # -0.18477343022823334
    0xBDBA7871,  # -0.09105003625154495
    0x00000000,  #  0.0
    0x3DA2FAFF,  #  0.07958029955625534
    0x3E24CAE3,  #  0.16093020141124725
    0x3E7C04DD,  #  0.24611230194354248
    0x3EAD033A,  #  0.33791524171829224
    0x3EE1A4B8,  #  0.44070982933044434
    0x3F1007AB,  #  0.5626170039176941
    0x3F3913B3,  #  0.7229568362236023
    0x3F800000,  #  1.0
]
NF4_CODEBOOK = np.array(_NF4_BITS, dtype=np.uint32).view(np.float32)
NF4_CODEBOOK.setflags(write=False)


def _check_shape(w):
    if w.ndim != 2:
        raise ValueError("NF4 weights must be 2-D [N, K]")
    if w.shape[1] % NF4_BLOCK:
        raise ValueError("K must be a multiple of 64 for NF4")


def nf4_pack(w):
    """Quantise float32 ``w [N, K]`` -> (codes uint8 [N, K/2], absmax float32 [N, K/64]).

    Follows the NF4 round-trip example on the "grouped-nf4-gemm 0.43.0"
    page (section "Try the packers and byte checks on CPU") with the
    readings listed in the module docstring.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    _check_shape(w)
    n, k = w.shape
    blocks = w.reshape(n, k // NF4_BLOCK, NF4_BLOCK)
    absmax = np.abs(blocks).max(axis=2).astype(np.float32)           # [N, K/64]
    safe = np.where(absmax == 0, np.float32(1), absmax)
    y = (blocks / safe[:, :, None]).astype(np.float32)               # fp32 division
    # nearest codebook entry; argmin returns the first (lower) index on ties
    dist = np.abs(y.astype(np.float64)[..., None] - NF4_CODEBOOK.astype(np.float64))
    codes = np.argmin(dist, axis=-1).astype(np.uint8)                 # [N, K/64, 64]
    codes[absmax == 0] = 7
    codes = codes.reshape(n, k)
    packed = ((codes[:, 0::2] << 4) | codes[:, 1::2]).astype(np.uint8)
    return packed, absmax


def nf4_decode(packed, absmax):
    """Decode (codes uint8 [N, K/2], absmax float32 [N, K/64]) -> float32 [N, K].

    Each weight is ``float32(q[code] * absmax[n, k // 64])``.
    """
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    n, half = packed.shape
    k = half * 2
    if absmax.shape != (n, k // NF4_BLOCK):
        raise ValueError("absmax must be [N, K/64]")
    codes = np.empty((n, k), dtype=np.uint8)
    codes[:, 0::2] = packed >> 4          # element 2j: high nibble
    codes[:, 1::2] = packed & 0x0F        # element 2j+1: low nibble
    q = NF4_CODEBOOK[codes]                                           # float32
    a = np.repeat(absmax, NF4_BLOCK, axis=1)                          # float32
    return (q * a).astype(np.float32)                                 # fp32 RNE multiply

