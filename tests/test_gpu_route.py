"""gq_route_sort on the GPU against the oracle's stable grouping, bit for
bit, on the routings of every workload plus the degenerate cases."""

import numpy as np
import pytest
import torch

import bit_grouped_moe_amd as gq
import oracle
import workloads as wl
from tests.gpu_common import device, say, to_dev

pytestmark = pytest.mark.gpu


def _check(ids, E, tile_m=256):
    dev = device()
    say("route_sort", ids.shape, E, tile_m)
    r = gq.gq_route_sort(to_dev(ids.astype(np.int32), dev), E, tile_m)
    torch.cuda.synchronize()
    off, sp, tiles = oracle.route_sort(ids, E, tile_m)
    n = int(r.num_tiles.item())
    assert np.array_equal(r.expert_offsets.cpu().numpy(), off)
    assert np.array_equal(r.sorted_pairs.cpu().numpy(), sp)
    t = r.tiles.cpu().numpy()
    assert n == len(tiles)
    assert np.array_equal(t[:n], tiles)
    assert np.all(t[n:] == -1)


def _cases():
    return {
        "tiny": (wl.route_uniform(wl.rng(wl.CFG_TINY, wl.S_ROUTE), 16, 4, 2), 4),
        "qwen_decode_m1": (wl.route_uniform(wl.rng(wl.CFG_QWEN_DECODE, wl.S_ROUTE), 1, 128, 8), 128),
        "qwen_decode_m4": (wl.route_uniform(wl.rng(wl.CFG_QWEN_DECODE, wl.S_ROUTE), 4, 128, 8), 128),
        "qwen_prefill_zipf": (wl.route_zipf(wl.rng(wl.CFG_QWEN_PREFILL, wl.S_ROUTE), 4096, 128, 8),
                              128),
        "gptoss_m2048": (wl.route_uniform(wl.rng(wl.CFG_GPTOSS, wl.S_ROUTE), 2048, 32, 4), 32),
        "qwen_dgrad_pairs": (wl.route_uniform(wl.rng(wl.CFG_QWEN_DGRAD, wl.S_ROUTE), 2048, 128, 8)
                             .reshape(-1, 1), 128),
    }


@pytest.mark.parametrize("name", list(_cases()))
def test_workload_routings(name):
    ids, E = _cases()[name]
    _check(ids, E)


@pytest.mark.parametrize("tile_m", [1, 7, 32, 256, 4096])
def test_tile_sizes(tile_m):
    ids = wl.route_zipf(wl.rng(9, 3), 500, 40, 3)
    _check(ids, 40, tile_m)


def test_degenerate():
    g = np.random.default_rng(0)
    _check(np.zeros((0, 8), dtype=np.int32), 128)                          # no pairs
    _check(np.full((300, 2), 5, dtype=np.int32), 8)                        # all on one expert
    ids = g.integers(-3, 11, (777, 3)).astype(np.int32)                    # dropped ids
    _check(ids, 8)
    _check(g.integers(0, 1, (50, 1)).astype(np.int32), 1)                  # E = 1
    _check(g.integers(0, 1024, (40, 4)).astype(np.int32), 1024)            # E = 1024, most empty
    _check(g.integers(0, 16, (16385, 3)).astype(np.int32), 16)             # two LDS chunks
    _check(g.integers(-2, 64, (9000, 8)).astype(np.int32), 64)             # three chunks, dropped
    _check(np.full((1, 1), -1, dtype=np.int32), 4)                          # only a dropped pair
