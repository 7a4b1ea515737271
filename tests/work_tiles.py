"""Expected FFN work list, for checking the library's moe_permute output.

Grouping the (token, expert) pairs by expert ("Strata" page, sec. 2.3: tokens
that picked the same expert share one fetch of its weights) gives each expert
a run of consecutive sorted rows; that much is the method, and the oracle's
permutation computes it.  The library hands each run to its FFN kernels in
tiles of at most 16 rows.  The tile format is the library's own, so this
checker lives with the tests, not in the oracle: per expert in ascending id,
per tile in row order, the int32 entry
    [expert, first row, rows, index of the tile among the expert's tiles,
     token of each row ..., then the token of the tile's first row repeated],
built with plain loops from the oracle's counts, offsets and sorted pairs.
"""
from __future__ import annotations

import numpy as np

import oracle


def expected_work_list(ids: np.ndarray, E: int, k: int, tile: int = 16) -> np.ndarray:
    perm = oracle.permute(ids, E)
    counts, offsets, sp = perm["counts"], perm["offsets"], perm["sorted_pairs"]
    out = []
    for e in range(E):
        for start in range(0, int(counts[e]), tile):
            row0 = int(offsets[e]) + start
            rows = min(tile, int(counts[e]) - start)
            toks = [int(sp[row0 + j]) // k for j in range(rows)]
            toks += [toks[0]] * (tile - rows)
            out.append([e, row0, rows, start // tile] + toks)
    return np.array(out, dtype=np.int32).reshape(-1, tile + 4)
