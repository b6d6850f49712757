"""fp64 oracle of the vocab-parallel LM head + cross-entropy (test
infrastructure only).

The logits of [TP-block] sec. 4 come from the output layer: a linear map of
the final hidden states h [N, H] by the [V, H] output embedding, split by
vocab like the input embedding of sec. 3 -- rank r holds rows [v0, v0 + V_r)
and computes its logits slice z_r = h W_r^T (a column-parallel linear: the
full h on every rank, a vocab slice of the output). The loss is the
vocab-parallel cross-entropy of ``xent`` on those slices. Backward: per rank
dz_r = (softmax - onehot) * dloss restricted to its columns (``xent``), then
the linear's two gradients dW_r = dz_r^T h and the input gradient
dh = sum_r dz_r W_r -- a partial per rank, summed over the ranks (the
column-parallel input's reduction in the backward).
"""
from __future__ import annotations

import numpy as np

from . import xent

F64 = np.float64


def logits(h, w_r):
    """z_r = h W_r^T, [N, V_r]."""
    return np.asarray(h, F64) @ np.asarray(w_r, F64).T


def forward(h, w_shards, target, vocab_starts):
    """Loss [N] and what the backward needs: (loss, gmax, sum_exp, logits list)."""
    zs = [logits(h, w) for w in w_shards]
    loss, gmax, sum_exp = xent.vocab_parallel_xent(zs, target, vocab_starts)
    return loss, gmax, sum_exp, zs


def backward_shard(h, w_r, z_r, target, v0, gmax, sum_exp, dloss):
    """One rank's (dh partial [N, H], dW_r [V_r, H])."""
    dz = xent.vocab_parallel_xent_bwd(z_r, target, v0, gmax, sum_exp, dloss)
    return dz @ np.asarray(w_r, F64), dz.T @ np.asarray(h, F64)
