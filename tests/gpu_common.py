"""Helpers for the GPU parity tests (oracle on the host, HIP path through
the C ABI).  Imported by tests only."""

import sys

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    gq.load_library()                       # raises if libgq.so is missing: no fallback
    return torch.device("cuda:0")


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu case]", *a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def bf16_to_host_f32(t):
    bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_to_f32(bits)


def bf16_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def packed_nf4_bank(g, E, N, K):
    """Oracle-packed NF4 bank of N(0, 0.02) weights: (codes [E,N,K/2], absmax [E,N,K/64])."""
    codes = np.empty((E, N, K // 2), dtype=np.uint8)
    absmax = np.empty((E, N, K // 64), dtype=np.float32)
    for e in range(E):
        w = g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        codes[e], absmax[e] = oracle.nf4_pack(w)
    return codes, absmax


def packed_mx_bank(g, E, N, K):
    blocks = np.empty((E, N, K // 32, 16), dtype=np.uint8)
    scales = np.empty((E, N, K // 32), dtype=np.uint8)
    for e in range(E):
        w = g.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        blocks[e], scales[e] = oracle.mxfp4_pack(w)
    return blocks, scales


class LazyDecoded:
    """Oracle decode of one expert at a time, cached (callable e -> [N, K] float32)."""

    def __init__(self, fmt, a, b):
        self.fmt, self.a, self.b, self.cache = fmt, a, b, {}

    def __call__(self, e):
        if e not in self.cache:
            if self.fmt == "nf4":
                self.cache[e] = oracle.nf4_decode(self.a[e], self.b[e])
            else:
                self.cache[e] = oracle.mxfp4_decode(self.a[e], self.b[e])
        return self.cache[e]


def assert_slices(y_gpu_f32, y_ref, pair_expert, E, experts=None):
    pe = np.asarray(pair_expert).reshape(-1)
    if experts is not None:
        keep = np.isin(pe, list(experts))
        y_gpu_f32, y_ref, pe = y_gpu_f32[keep], y_ref[keep], pe[keep]
    ok, errs = oracle.compare_slices(y_gpu_f32, y_ref, pe, E)
    worst = max([v for v in errs.values() if isinstance(v, float)] or [0.0])
    assert ok, f"per-expert rel-L2 above {oracle.REL_L2_TOL}: worst {worst}; {errs}"
    return worst


def assert_rows(y_gpu_f32, y_ref, tol=None, what=""):
    """Per-row relative L2 <= tol (default: the per-slice tolerance) for
    every row of a checked set; a row whose reference is exactly zero must
    be exactly zero.  A single wrong row in a large expert slice barely
    moves the slice error; this catches it."""
    tol = oracle.REL_L2_TOL if tol is None else tol
    y_ref = np.asarray(y_ref, dtype=np.float64)
    d = np.asarray(y_gpu_f32, dtype=np.float64) - y_ref
    nr = np.linalg.norm(y_ref, axis=1)
    nd = np.linalg.norm(d, axis=1)
    zero = nr == 0.0
    assert not np.any(nd[zero]), f"{what}: rows {np.nonzero(zero & (nd > 0))[0][:8]} should be 0"
    err = nd[~zero] / nr[~zero]
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, (f"{what}: per-row rel-L2 {worst} above {tol} "
                          f"(row {np.nonzero(~zero)[0][int(err.argmax())]})")
    return worst


def plus_zero(bits):
    """bf16 bit patterns with -0 mapped to +0.  A one-hot probe multiplies a
    decoded weight by 1 and adds zero products: IEEE round-to-nearest gives
    +0 when that weight is -0 (e2m1 code 8), so probes compare up to the
    sign of zero."""
    b = np.asarray(bits, dtype=np.uint16).copy()
    b[b == 0x8000] = 0
    return b


def unpermute_split(codes, scales, K):
    """Natural-order (hi, lo, s_hi, s_lo) from the split kernel's layout:
    per 64-k step, 128 bytes = hi then lo (64 each); in each, bytes
    [32h, 32h + 32) hold elements 16h + [0, 16) of k block 2s, then of
    block 2s + 1; scales per step s_hi(2s), s_lo(2s), s_hi(2s+1), s_lo(2s+1)."""
    rows = codes.shape[0]
    kp = codes.shape[1] // 2
    c = codes.reshape(rows, kp // 64, 2, 2, 2, 16)        # [row, step, term, h, block, i]
    c = c.transpose(0, 1, 2, 4, 3, 5)                     # [row, step, term, block, h, i]
    hi = c[:, :, 0].reshape(rows, kp)[:, :K]
    lo = c[:, :, 1].reshape(rows, kp)[:, :K]
    s = scales.reshape(rows, kp // 64, 2, 2)              # [row, step, block, term]
    s_hi = s[:, :, :, 0].reshape(rows, kp // 32)[:, :K // 32]
    s_lo = s[:, :, :, 1].reshape(rows, kp // 32)[:, :K // 32]
    return hi, lo, s_hi, s_lo


def same_codes(a, b):
    """e4m3 codes equal up to the sign of zero (0x00 vs 0x80 hold the same value)."""
    a = np.where(a == 0x80, 0, a)
    b = np.where(b == 0x80, 0, b)
    return np.array_equal(a, b)
