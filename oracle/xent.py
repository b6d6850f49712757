"""fp64 oracle of the vocab-parallel cross-entropy (test infrastructure only).

[TP-block] sec. 4: the logits [N, V] are split by vocab into R contiguous
shards [N, V/R]; shard r holds vocab ids [r*V/R, (r+1)*V/R). The loss is
formed without gathering the logits, from three small reductions:

  1. local row max, then a global MAX over shards;
  2. on each shard, exp(z - global max) summed over its columns, and the
     max-subtracted target logit, which is non-zero only on the shard that
     owns the target id; both are then SUMmed over shards;
  3. loss = log(sum_exp) - predicted (= -log softmax at the target).

The backward is local to each shard: dz = (softmax - onehot(target)) * dloss.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def shard_ranges(vocab, R):
    n = vocab // R
    return [(r * n, (r + 1) * n) for r in range(R)]


def local_max(z_r):
    """Step 1, per shard: row max over the shard's columns."""
    return np.asarray(z_r, F64).max(axis=1)


def local_sums(z_r, target, v0, gmax):
    """Step 2, per shard: (sum_j exp(z - gmax), predicted) where predicted is
    z[target] - gmax when the target id lies in [v0, v0 + V_r), else 0."""
    z = np.asarray(z_r, F64)
    sum_exp = np.exp(z - gmax[:, None]).sum(axis=1)
    n, vr = z.shape
    local = target - v0
    own = (local >= 0) & (local < vr)
    pred = np.zeros(n, F64)
    rows = np.nonzero(own)[0]
    pred[rows] = z[rows, local[rows]] - gmax[rows]
    return sum_exp, pred


def vocab_parallel_xent(shards, target, vocab_starts):
    """Loss [N] from the list of shard logits, in the order of the page's
    three reductions. Returns (loss, gmax, sum_exp)."""
    gmax = np.max(np.stack([local_max(z) for z in shards]), axis=0)        # all-reduce MAX
    parts = [local_sums(z, target, v0, gmax) for z, v0 in zip(shards, vocab_starts)]
    predicted = np.sum([p for _, p in parts], axis=0)                     # all-reduce SUM
    sum_exp = np.sum([s for s, _ in parts], axis=0)                       # all-reduce SUM
    loss = np.log(sum_exp) - predicted
    return loss, gmax, sum_exp


def vocab_parallel_xent_bwd(z_r, target, v0, gmax, sum_exp, dloss):
    """Shard-local gradient: dz = (exp(z - gmax) / sum_exp - onehot) * dloss."""
    z = np.asarray(z_r, F64)
    p = np.exp(z - gmax[:, None]) / sum_exp[:, None]
    n, vr = z.shape
    local = target - v0
    rows = np.nonzero((local >= 0) & (local < vr))[0]
    p[rows, local[rows]] -= 1.0
    return p * np.asarray(dloss, F64)[:, None]
