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
* ``tiles``: the GEMM work list.  The pages fix no tiling and many are
  correct, so the oracle does not prescribe one: ``check_tiles`` states what
  any valid list satisfies (experts ascending; each expert's padded rows
  ``[padded_offsets[e], padded_offsets[e+1])`` covered by consecutive tiles
  in row order, without gaps or overlaps; every tile a positive multiple of
  ``row_pad`` rows and at most ``tile_rows``; no tile for an expert without
  rows), and ``route`` returns the simplest such list (greedy tiles of
  ``tile_rows`` rows, the last one shorter) as one example of it.
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
    for e in range(E):
        r = padded_offsets[e]
        while r < padded_offsets[e + 1]:
            n = min(tile_rows // row_pad * row_pad, padded_offsets[e + 1] - r)
            tiles.append((e, r, n))
            r += n
    i32 = np.int32
    return Routing(
        counts=np.array(counts, dtype=i32),
        offsets=np.array(offsets, dtype=i32),
        padded_offsets=np.array(padded_offsets, dtype=i32),
        sorted_ids=np.array(sorted_ids, dtype=i32),
        pos=np.array(pos, dtype=i32),
        tiles=np.array(tiles, dtype=i32).reshape(-1, 3),
    )


def check_tiles(tiles, n_tiles, padded_offsets, num_experts, row_pad, tile_rows):
    """Problems of a GEMM tile list (empty if it is valid).

    ``tiles``: int [n, >=3] rows (expert, first_row, n_rows); ``n_tiles``: the
    count the producer reports.  Valid means: ``n_tiles == len(tiles)``; the
    experts are ascending; for each expert the tiles start at
    ``padded_offsets[e]``, each begins where the previous one ended, and the
    last ends at ``padded_offsets[e+1]``; every tile has a positive multiple
    of ``row_pad`` rows, at most ``tile_rows``; an expert with no rows has no
    tile."""
    problems = []
    t = np.asarray(tiles).reshape(-1, np.shape(tiles)[-1] if np.ndim(tiles) == 2 else 3)
    po = [int(v) for v in padded_offsets]
    if int(n_tiles) != len(t):
        problems.append(f"tile count {int(n_tiles)} != {len(t)} tiles listed")
    by_expert = {}
    prev_e = -1
    for i, row in enumerate(t):
        e, r0, n = int(row[0]), int(row[1]), int(row[2])
        if not 0 <= e < num_experts:
            problems.append(f"tile {i}: expert {e} out of range")
            continue
        if e < prev_e:
            problems.append(f"tile {i}: expert {e} after expert {prev_e}")
        prev_e = e
        if n <= 0 or n % row_pad or n > tile_rows:
            problems.append(f"tile {i}: {n} rows (need a positive multiple of {row_pad}, at most {tile_rows})")
        by_expert.setdefault(e, []).append((r0, n))
    for e in range(num_experts):
        lo, hi = po[e], po[e + 1]
        segs = by_expert.get(e, [])
        if lo == hi:
            if segs:
                problems.append(f"expert {e} has no rows but {len(segs)} tiles")
            continue
        r = lo
        for r0, n in segs:
            if r0 != r:
                problems.append(f"expert {e}: tile starts at row {r0}, expected {r}")
            r = r0 + n
        if r != hi:
            problems.append(f"expert {e}: tiles end at row {r}, expected {hi}")
    return problems
