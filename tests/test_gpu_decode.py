"""Decode probes on the GPU against the oracle, bit for bit (float32 and
bf16), over every code byte, every e8m0 scale byte and edge-case absmax."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
from tests.gpu_common import bf16_bits, device, say, to_dev

pytestmark = pytest.mark.gpu


def _f32_bits(t):
    return t.cpu().numpy().view(np.uint32)


def test_nf4_decode_every_byte_and_edge_absmax():
    dev = device()
    absmax_vals = np.array([1.0, 0.5, 0.0371, 2.0 ** -20, 1e-39, 3.0e38, 0.0, -0.25, 7.0e-3,
                            123.456], dtype=np.float32)
    rows = len(absmax_vals)
    codes = np.tile(np.arange(256, dtype=np.uint8), (rows, 1))          # K = 512
    absmax = np.repeat(absmax_vals[:, None], 8, axis=1).astype(np.float32)
    say("nf4_decode every byte", rows)
    f, b = gq.gq_nf4_decode(to_dev(codes, dev), to_dev(absmax, dev))
    torch.cuda.synchronize()
    ref = oracle.nf4_decode(codes, absmax)
    assert np.array_equal(_f32_bits(f), ref.view(np.uint32))
    assert np.array_equal(bf16_bits(b), oracle.f32_to_bf16_rne(ref))


def test_nf4_decode_packed_gaussian():
    dev = device()
    g = np.random.default_rng(3)
    w = g.standard_normal((300, 1024)).astype(np.float32) * np.float32(0.02)
    codes, absmax = oracle.nf4_pack(w)
    say("nf4_decode gaussian", codes.shape)
    f, b = gq.gq_nf4_decode(to_dev(codes, dev), to_dev(absmax, dev))
    torch.cuda.synchronize()
    ref = oracle.nf4_decode(codes, absmax)
    assert np.array_equal(_f32_bits(f), ref.view(np.uint32))
    assert np.array_equal(bf16_bits(b), oracle.f32_to_bf16_rne(ref))


def test_mxfp4_decode_every_byte_every_scale():
    dev = device()
    # 256 rows (one per scale byte) x 16 blocks (every byte value once per row)
    blocks = np.tile(np.arange(256, dtype=np.uint8).reshape(16, 16), (256, 1, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, axis=1)
    say("mxfp4_decode every byte every scale")
    f, b = gq.gq_mxfp4_decode(to_dev(blocks, dev), to_dev(scales, dev))
    torch.cuda.synchronize()
    ref = oracle.mxfp4_decode(blocks, scales)
    got = f.cpu().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])
    gb = bf16_bits(b)
    rb = oracle.f32_to_bf16_rne(ref)
    assert np.all(np.isnan(oracle.bf16_to_f32(gb)[nan]))
    assert np.array_equal(gb[~nan], rb[~nan])


def test_mxfp4_decode_packed_gaussian():
    dev = device()
    g = np.random.default_rng(4)
    w = g.standard_normal((200, 2880)).astype(np.float32) * np.float32(0.02)
    blocks, scales = oracle.mxfp4_pack(w)
    say("mxfp4_decode gaussian", blocks.shape)
    f, b = gq.gq_mxfp4_decode(to_dev(blocks, dev), to_dev(scales, dev))
    torch.cuda.synchronize()
    ref = oracle.mxfp4_decode(blocks, scales)
    assert np.array_equal(_f32_bits(f), ref.view(np.uint32))
    assert np.array_equal(bf16_bits(b), oracle.f32_to_bf16_rne(ref))
