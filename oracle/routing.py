"""Routing stage of the fused MoE, integer only (oracle).

TEST INFRASTRUCTURE ONLY.

The b12x README ("Using it") binds caller-supplied ``topk_ids`` and
``topk_weights`` to fused_moe, and ("What's in here") describes a routed-expert
FFN run over per-expert work.  The pages do not define the routing buffers;
this module states the canonical form that the grouped GEMMs consume, so that
the GPU stage can be compared with it bit for bit:

* pair ``p = t*k + j`` is slot ``j`` of token ``t``; its expert is
  ``topk_ids[t, j]``; an id outside ``[0, E)`` drops the pair (it contributes
  nothing to the output);
* ``counts[e]``  = number of valid pairs routed to ``e``;
* ``offsets``    = exclusive prefix sum of ``counts`` (length E+1);
* ``padded[e]``  = ``counts[e]`` rounded up to a multiple of ``row_pad``;
  ``padded_offsets`` = exclusive prefix sum of ``padded`` (length E+1);
* ``sorted_ids[padded_offsets[e] + r]`` = the r-th valid pair routed to ``e``
  in ascending ``p`` (a stable sort by expert); padding rows hold -1;
* ``pos[p]`` = the row of pair ``p`` in ``sorted_ids``, or -1 if dropped;
* ``tiles``: for each expert in ascending order, the rows
  ``[padded_offsets[e], padded_offsets[e+1])`` as blocks of ``row_pad`` rows,
  split into the fewest tiles of at most ``tile_rows`` rows with the block
  counts as equal as possible (the first ``nb mod n`` tiles take one block
  more), as ``(expert, first_row, n_rows)``.
"""
from dataclasses import dataclass

import numpy as np


@dataclass
class Routing:
    counts: np.ndarray          # int32 [E]
    offsets: np.ndarray         # int32 [E+1]
    padded_offsets: np.ndarray  # int32 [E+1]
    sorted_ids: np.ndarray      # int32 [padded_offsets[E]]
    pos: np.ndarray             # int32 [P]
    tiles: np.ndarray           # int32 [n_tiles, 3]


def route(topk_ids, num_experts, row_pad, tile_rows):
    ids = np.asarray(topk_ids).reshape(-1)
    n_pairs = ids.size
    E = int(num_experts)
    counts = [0] * E
    for p in range(n_pairs):
        e = int(ids[p])
        if 0 <= e < E:
            counts[e] += 1
    offsets = [0] * (E + 1)
    padded_offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
        padded = -(-counts[e] // row_pad) * row_pad
        padded_offsets[e + 1] = padded_offsets[e] + padded
    sorted_ids = [-1] * padded_offsets[E]
    pos = [-1] * n_pairs
    filled = [0] * E
    for p in range(n_pairs):
        e = int(ids[p])
        if 0 <= e < E:
            row = padded_offsets[e] + filled[e]
            sorted_ids[row] = p
            pos[p] = row
            filled[e] += 1
    tiles = []
    max_blocks = tile_rows // row_pad
    for e in range(E):
        n_blocks = (padded_offsets[e + 1] - padded_offsets[e]) // row_pad
        n_tiles = -(-n_blocks // max_blocks)
        r = padded_offsets[e]
        for i in range(n_tiles):
            blocks = n_blocks // n_tiles + (1 if i < n_blocks % n_tiles else 0)
            tiles.append((e, r, blocks * row_pad))
            r += blocks * row_pad
    i32 = np.int32
    return Routing(
        counts=np.array(counts, dtype=i32),
        offsets=np.array(offsets, dtype=i32),
        padded_offsets=np.array(padded_offsets, dtype=i32),
        sorted_ids=np.array(sorted_ids, dtype=i32),
        pos=np.array(pos, dtype=i32),
        tiles=np.array(tiles, dtype=i32).reshape(-1, 3),
    )
