"""Routing: stable counting sort of the routed rows by expert.

[P3] "Key source snippets": pre_dispatch receives topk_ids / topk_weights per
token and hands them to the expert kernel together with the packed tokens.
The pages do not print the permutation itself; the reading taken here is the
plain one:

  routed row r = t*k + j (token t, slot j) is valid iff 0 <= ids[t, j] < E;
  counts[e]   = number of valid rows with expert e;
  offsets     = exclusive prefix sum of counts (length E+1);
  sorted_rows = the valid r ordered by (expert, r)   -- a stable sort;
  pos[r]      = index of r in sorted_rows, or -1 for an invalid row.

Ids outside [0, E) (e.g. -1 for a masked slot) are skipped; a token that names
the same expert twice contributes two separate rows.
"""
from __future__ import annotations

import numpy as np


def route(topk_ids, num_experts: int):
    """Counting sort written out: one counting pass, a prefix sum, one placing pass.

    Returns (counts int32 [E], offsets int32 [E+1], sorted_rows int32 [n_valid],
    pos int32 [T*k]).
    """
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    R = ids.shape[0]
    E = int(num_experts)
    counts = np.zeros(E, dtype=np.int64)
    for r in range(R):
        e = ids[r]
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:E].copy()
    sorted_rows = np.empty(offsets[E], dtype=np.int64)
    pos = np.full(R, -1, dtype=np.int64)
    for r in range(R):                       # ascending r: ties keep their order
        e = ids[r]
        if 0 <= e < E:
            sorted_rows[cursor[e]] = r
            pos[r] = cursor[e]
            cursor[e] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_rows.astype(np.int32), pos.astype(np.int32))
