"""Token-to-expert grouping for the oracle (test infrastructure only).

The pages require every active expert to run in one GPU launch
("grouped-nf4-gemm 0.43.0", page header: one launch for the active
experts) and describe the routing tensor as a contiguous int array
``[M, top_k]`` of expert ids whose results land in ``[M, top_k, N]``
("flashrt/grouped-moe-gemv", section "Functions").  How the pairs are
grouped is left open; the reading taken is a stable counting sort:

* pair index ``p = token * top_k + slot`` (row-major flattening);
* ``offsets[e]`` = number of valid pairs routed to experts ``< e``;
  ``offsets[E]`` = number of valid pairs;
* ``sorted_pairs`` lists, expert by expert in ascending order, the pair
  indices routed to that expert in ascending ``p``; pairs whose id is
  outside ``[0, E)`` are dropped and listed last, ascending;
* ``tiles`` lists ``(expert, start)`` for every ``tile_m``-row slice of each
  expert's segment, experts ascending, ``start`` an index into
  ``sorted_pairs``.

Exactly one answer satisfies this definition, so the HIP result must match
it bit for bit.
"""

import numpy as np

__all__ = ["route_sort"]


def route_sort(topk_ids, num_experts, tile_m):
    """Return (offsets int32 [E+1], sorted_pairs int32 [P], tiles int32 [T, 2])."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    E = int(num_experts)
    valid = (ids >= 0) & (ids < E)
    offsets = [0]
    sorted_pairs = []
    tiles = []
    for e in range(E):
        members = [p for p in np.nonzero(ids == e)[0].tolist()]   # ascending p
        for m0 in range(0, len(members), tile_m):
            tiles.append((e, len(sorted_pairs) + m0))
        sorted_pairs.extend(members)
        offsets.append(len(sorted_pairs))
    sorted_pairs.extend(np.nonzero(~valid)[0].tolist())
    return (np.array(offsets, dtype=np.int32),
            np.array(sorted_pairs, dtype=np.int32),
            np.array(tiles, dtype=np.int32).reshape(-1, 2))
