"""Pins for the oracle's MXFP4 packer / decoder.

* e2m1 values against the OCP MX v1.0 magnitude list (hand-typed);
* exhaustive decode of all 16 codes x 256 scale bytes against math.ldexp;
* the printed MXFP4 round-trip on the "grouped-nf4-gemm 0.43.0" page
  (section "Try the packers and byte checks on CPU"): shapes and relative
  error about 0.12; re-pack idempotency under the OCP scale rule;
* element rounding by brute force, the shared-exponent rule, nibble order.
"""

import math

import numpy as np

from oracle import E2M1_VALUES, mxfp4_pack, mxfp4_decode


def test_e2m1_values_match_spec(golden):
    want = golden["e2m1_values"]["values"]
    assert E2M1_VALUES.tolist() == want
    assert math.copysign(1.0, E2M1_VALUES[8]) == -1.0


def test_exhaustive_decode_against_ldexp():
    blocks = np.zeros((256, 1, 16), dtype=np.uint8)
    blocks[:, 0, :] = np.array([c | ((15 - c) << 4) for c in range(16)], dtype=np.uint8)
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    w = mxfp4_decode(blocks, scales)                                   # [256, 32]
    golden_vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for s in range(256):
        for j in range(16):
            for elem, code in ((2 * j, j), (2 * j + 1, 15 - j)):
                got = w[s, elem]
                if s == 255:
                    assert np.isnan(got)
                    continue
                mag = golden_vals[code & 7]
                ref = math.ldexp(mag, s - 127) * (-1.0 if code & 8 else 1.0)
                with np.errstate(over="ignore"):
                    ref32 = np.float32(ref)
                assert got == ref32 or (np.isinf(ref32) and got == ref32), (s, code)
                if ref32 == 0:
                    assert math.copysign(1.0, got) == math.copysign(1.0, ref)


def test_printed_roundtrip(golden):
    spec = golden["mxfp4_roundtrip"]
    for seed in range(3):
        w = np.random.default_rng(seed).standard_normal(spec["w_shape"]).astype(np.float32)
        blocks, scales = mxfp4_pack(w)
        assert list(blocks.shape) == spec["blocks_shape"] and blocks.dtype == np.uint8
        assert list(scales.shape) == spec["scales_shape"] and scales.dtype == np.uint8
        wq = mxfp4_decode(blocks, scales)
        assert wq.shape == w.shape
        rel = np.linalg.norm(wq - w) / np.linalg.norm(w)
        lo, hi = spec["rel_err_band"]
        assert lo <= rel <= hi, rel
        b2, s2 = mxfp4_pack(wq)
        assert np.array_equal(b2, blocks) and np.array_equal(s2, scales)


def test_shared_exponent_rule():
    g = np.random.default_rng(7)
    w = (g.standard_normal((64, 256)) * np.exp(g.uniform(-20, 20, (64, 1)))).astype(np.float32)
    _, scales = mxfp4_pack(w)
    amax = np.abs(w.reshape(64, 8, 32).astype(np.float64)).max(-1)
    x = scales.astype(np.int64) - 127
    # 2**(X+2) <= amax < 2**(X+3): the largest element scales into [4, 8)
    assert np.all(np.ldexp(1.0, x + 2) <= amax)
    assert np.all(amax < np.ldexp(1.0, x + 3))


def test_element_rounding_brute_force():
    g = np.random.default_rng(11)
    w = g.standard_normal((4, 64)).astype(np.float32)
    # plant exact ties: 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times the block scale
    w[0, :7] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    w[0, 7] = 7.9
    blocks, scales = mxfp4_pack(w)
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for n in range(4):
        for k in range(64):
            X = int(scales[n, k // 32]) - 127
            v = abs(float(w[n, k])) * math.ldexp(1.0, -X)
            v = min(v, 6.0)
            best = min(range(8), key=lambda i: (abs(v - mags[i]), i % 2, i))
            b = int(blocks[n, k // 32, (k % 32) // 2])
            code = b & 15 if k % 2 == 0 else b >> 4
            assert code & 7 == best, (n, k, v)
            assert (code >> 3) == int(np.signbit(w[n, k]))
    # the planted ties: scale is 2**(2-2)=1 for amax 7.9
    assert int(scales[0, 0]) == 127
    b = blocks[0, 0]
    codes = [b[j // 2] & 15 if j % 2 == 0 else b[j // 2] >> 4 for j in range(8)]
    assert [int(c) for c in codes] == [0, 2, 2, 4, 4, 6, 6, 7]


def test_nibble_order_golden(golden):
    g = golden["nibble_order"]
    codes = g["mxfp4_row_codes"]
    vals = [E2M1_VALUES[c] for c in codes]
    row = np.zeros(32, dtype=np.float32)
    row[: len(vals)] = vals
    row[31] = 6.0                                                    # pin the scale to 2**0
    blocks, scales = mxfp4_pack(row[None, :])
    assert int(scales[0, 0]) == 127
    assert blocks[0, 0, : len(g["mxfp4_row_bytes_prefix"])].tolist() == g["mxfp4_row_bytes_prefix"]


def test_zero_block_and_negative_zero():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 32] = -1e-30
    w[0, 33] = 1.0
    blocks, scales = mxfp4_pack(w)
    assert int(scales[0, 0]) == 0                                     # X = -127
    assert np.all(blocks[0, 0] == 0)
    assert int(blocks[0, 1, 0]) & 15 == 8                             # -0 keeps its sign bit
    out = mxfp4_decode(blocks, scales)
    assert out[0, 32] == 0.0 and math.copysign(1.0, out[0, 32]) == -1.0
