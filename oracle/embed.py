"""fp64 oracle of the vocab-parallel input embedding (test infrastructure only).

[TP-block] sec. 3: the [vocab, h] embedding table is split by vocab over the
R tensor-parallel ranks; rank r holds the contiguous rows [v0, v0 + V_r).
Each rank looks up only the token ids that fall in its range -- ids outside
it are masked before the lookup and their rows are zeroed after it -- and an
all-reduce then sums the R partial results, so every token gets exactly one
non-zero contribution.

The backward is the adjoint of that forward (the page prints the forward
only; this is the plain reading): the all-reduce's backward is the identity,
so every rank receives the full output gradient and adds the gradient row of
each token whose id lies in its range into that id's table row.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def shard_ranges(vocab, R):
    n = vocab // R
    return [(r * n, (r + 1) * n) for r in range(R)]


def embed_fwd(table_r, ids, v0):
    """One rank's masked lookup: row ids[t] - v0 of its table slice when the
    id lies in [v0, v0 + V_r), else a zero row. Returns [N, h] float64."""
    table = np.asarray(table_r, F64)
    vr, h = table.shape
    ids = np.asarray(ids, np.int64)
    local = ids - v0
    own = (local >= 0) & (local < vr)              # the mask
    masked = np.where(own, local, 0)               # masked ids look up row 0 ...
    out = table[masked]
    out[~own] = 0.0                                # ... and are zeroed after the lookup
    return out


def embed_fwd_sharded(tables, ids, vocab_starts):
    """The all-reduce: sum of every rank's masked lookup."""
    return np.sum([embed_fwd(t, ids, v0) for t, v0 in zip(tables, vocab_starts)], axis=0)


def embed_bwd(dout, ids, v0, v_local):
    """One rank's table gradient [V_r, h]: for each token t (in order) whose id
    lies in [v0, v0 + V_r), dout[t] is added to row ids[t] - v0."""
    g = np.asarray(dout, F64)
    ids = np.asarray(ids, np.int64)
    d = np.zeros((v_local, g.shape[1]), F64)
    for t in range(ids.shape[0]):
        v = int(ids[t]) - v0
        if 0 <= v < v_local:
            d[v] += g[t]
    return d
