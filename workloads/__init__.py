"""Seeded synthetic inputs shared by the tests and the benchmark.

This module draws numbers only; it contains none of the packing, decoding
or matmul arithmetic of the method.  Weights are drawn in float32 (packing
them is the oracle's job), activations are drawn in float32 and converted
to bf16 by torch (round to nearest even), routings and router weights are
drawn per token.  For very large banks, where packing on the host would
take minutes, ``random_nf4_bank`` / ``random_mxfp4_bank`` draw already
packed bytes directly from the distribution that packing N(0, 0.02)
weights produces; kernel time does not depend on the values.

Workload recipe (one ``numpy.random.Generator(PCG64(SeedSequence([cfg,
stream])))`` per stream; cfg 0..4 are the five workloads below, stream 0
gate_up weights, 1 down weights, 2 activations, 3 routing, 4 router
logits, 5 down-projection inputs / output gradients):

* tiny NF4 grouped GEMM: E=4, W [256, 512], 16 tokens, top-2 uniform;
* Qwen3-30B-A3B-shaped NF4 decode: E=128, gate_up W [1536, 2048], down
  W [2048, 768], M=1 and M=4, top-8 distinct uniform;
* Qwen3-30B-A3B-shaped NF4 prefill: same experts, M=4096, top-8 with
  Zipf(1.1) expert popularity, router weights softmax(N(0,1) logits);
* gpt-oss-20b-shaped MXFP4: E=32, gate_up W [5760, 2880], down
  W [2880, 2880], M=1 and M=2048, top-4 uniform;
* NF4 dgrad at Qwen3-30B-A3B shapes: M=2048 top-8 uniform, dY N(0,1).
"""

import numpy as np

__all__ = [
    "CFG_TINY", "CFG_QWEN_DECODE", "CFG_QWEN_PREFILL", "CFG_GPTOSS", "CFG_QWEN_DGRAD",
    "S_W_GATE_UP", "S_W_DOWN", "S_X", "S_ROUTE", "S_LOGITS", "S_DOWN_IN",
    "QWEN", "GPTOSS", "TINY",
    "rng", "draw_weights", "draw_bf16", "route_uniform", "route_zipf", "router_weights",
    "random_nf4_bank", "random_mxfp4_bank",
]

CFG_TINY, CFG_QWEN_DECODE, CFG_QWEN_PREFILL, CFG_GPTOSS, CFG_QWEN_DGRAD = range(5)
S_W_GATE_UP, S_W_DOWN, S_X, S_ROUTE, S_LOGITS, S_DOWN_IN = range(6)

# expert shapes: projection -> (N, K)
QWEN = {"E": 128, "gate_up": (1536, 2048), "down": (2048, 768), "topk": 8}
GPTOSS = {"E": 32, "gate_up": (5760, 2880), "down": (2880, 2880), "topk": 4}
TINY = {"E": 4, "gate_up": (256, 512), "topk": 2, "M": 16}


def rng(cfg, stream):
    """Independent generator for (workload, stream)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(cfg), int(stream)])))


def draw_weights(g, E, N, K, std=0.02):
    """float32 [E, N, K] ~ N(0, std^2), drawn expert by expert."""
    out = np.empty((E, N, K), dtype=np.float32)
    for e in range(E):
        out[e] = g.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    return out


def draw_bf16(g, shape, std=1.0):
    """uint16 bf16 bit patterns of float32 N(0, std^2) draws (torch RNE cast)."""
    import torch
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def route_uniform(g, M, E, k):
    """int32 [M, k]: per token, k distinct experts chosen uniformly."""
    out = np.empty((M, k), dtype=np.int32)
    for t in range(M):
        out[t] = np.argsort(g.random(E))[:k]
    return out


def route_zipf(g, M, E, k, s=1.1):
    """int32 [M, k]: per token, k distinct experts drawn without replacement
    with popularity p_e proportional to (e+1)^-s (Gumbel top-k, which is
    sequential weighted sampling without replacement)."""
    logp = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(g.random((M, E))))
    keys = logp[None, :] + gumbel
    return np.argsort(-keys, axis=1)[:, :k].astype(np.int32)


def router_weights(g, M, k):
    """float32 [M, k]: softmax over each token's k N(0,1) logits (float64 -> float32)."""
    z = g.standard_normal((M, k))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def _max_abs_normal(u, n):
    """Inverse CDF of max of n iid |N(0,1)| at uniform u (torch tensors),
    evaluated in float64 so that u**(1/n) stays below 1."""
    import torch
    v = u.to(torch.float64).clamp(1e-12, 1.0 - 1e-12).pow(1.0 / n)
    return torch.erfinv(v) * (2.0 ** 0.5)


def random_nf4_bank(E, N, K, device, seed, std=0.02):
    """Directly drawn NF4-packed bank (torch tensors on ``device``):
    codes uint8 [E, N, K/2] with independent uniform nibbles (NF4's
    quantile construction makes the codes of Gaussian weights close to
    uniform), absmax float32 [E, N, K/64] = std * (max of 64 |N(0,1)|)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    codes = torch.randint(0, 256, (E, N, K // 2), dtype=torch.uint8, device=device, generator=gen)
    u = torch.rand((E, N, K // 64), device=device, generator=gen, dtype=torch.float32)
    absmax = (_max_abs_normal(u, 64) * std).to(torch.float32)
    return codes, absmax


def random_mxfp4_bank(E, N, K, device, seed):
    """Directly drawn MXFP4 bank: blocks uint8 [E, N, K/32, 16] uniform
    bytes, scales uint8 [E, N, K/32] drawn from {119, 120, 121} with
    probabilities {0.02, 0.925, 0.055} (the e8m0 exponents that blocks of
    32 N(0, 0.02) weights receive)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    blocks = torch.randint(0, 256, (E, N, K // 32, 16), dtype=torch.uint8, device=device,
                           generator=gen)
    u = torch.rand((E, N, K // 32), device=device, generator=gen)
    scales = torch.full_like(u, 120, dtype=torch.uint8)
    scales[u < 0.02] = 119
    scales[u > 1 - 0.055] = 121
    return blocks, scales
