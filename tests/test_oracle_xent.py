"""Pins for the vocab-parallel cross-entropy oracle (CPU only)."""
import math

import numpy as np
from scipy.special import logsumexp, softmax

from oracle import xent as ox


def _shards(z, R):
    V = z.shape[1]
    return [z[:, a:b] for a, b in ox.shard_ranges(V, R)], [a for a, _ in ox.shard_ranges(V, R)]


def test_sharded_loss_equals_full_logsumexp_minus_target():
    rng = np.random.default_rng(1)
    N, V, R = 64, 96, 8
    z = rng.normal(size=(N, V)) * 4
    y = rng.integers(0, V, N)
    y[:R] = [r * (V // R) for r in range(R)]             # first id of each shard
    y[R:2 * R] = [(r + 1) * (V // R) - 1 for r in range(R)]  # last id of each shard
    sh, v0 = _shards(z, R)
    loss, gmax, sexp = ox.vocab_parallel_xent(sh, y, v0)
    ref = logsumexp(z, axis=1) - z[np.arange(N), y]
    assert np.max(np.abs(loss - ref)) < 1e-12
    assert np.array_equal(gmax, z.max(1))
    # same value for any shard count that divides V
    for R2 in (1, 2, 3):
        l2, _, _ = ox.vocab_parallel_xent(*_shards(z, R2)[:1], y, _shards(z, R2)[1])
        assert np.max(np.abs(l2 - ref)) < 1e-12


def test_gradient_is_softmax_minus_onehot_and_rows_sum_to_zero():
    rng = np.random.default_rng(2)
    N, V, R = 16, 40, 4
    z = rng.normal(size=(N, V))
    y = rng.integers(0, V, N)
    dl = rng.normal(size=N)
    sh, v0 = _shards(z, R)
    _, gmax, sexp = ox.vocab_parallel_xent(sh, y, v0)
    dz = np.concatenate([ox.vocab_parallel_xent_bwd(s, y, a, gmax, sexp, dl) for s, a in zip(sh, v0)], 1)
    onehot = np.zeros_like(z)
    onehot[np.arange(N), y] = 1
    assert np.max(np.abs(dz - (softmax(z, axis=1) - onehot) * dl[:, None])) < 1e-15
    assert np.max(np.abs(dz.sum(1))) < 1e-14


def test_gradient_matches_central_differences():
    rng = np.random.default_rng(3)
    N, V, R = 3, 12, 3
    z = rng.normal(size=(N, V))
    y = np.array([0, 5, 11])
    wts = rng.normal(size=N)

    def L(zz):
        s, a = _shards(zz, R)
        return float((ox.vocab_parallel_xent(s, y, a)[0] * wts).sum())

    s, a = _shards(z, R)
    _, gmax, sexp = ox.vocab_parallel_xent(s, y, a)
    dz = np.concatenate([ox.vocab_parallel_xent_bwd(q, y, b, gmax, sexp, wts) for q, b in zip(s, a)], 1)
    h = 1e-6
    for idx in np.ndindex(N, V):
        zp = z.copy(); zp[idx] += h
        zm = z.copy(); zm[idx] -= h
        assert abs((L(zp) - L(zm)) / (2 * h) - dz[idx]) < 1e-8


def test_all_equal_logits():
    N, V, R = 5, 32, 4
    z = np.full((N, V), 0.75)
    y = np.array([0, 7, 8, 31, 16])
    dl = np.full(N, 0.5)
    sh, v0 = _shards(z, R)
    loss, gmax, sexp = ox.vocab_parallel_xent(sh, y, v0)
    assert np.max(np.abs(loss - math.log(V))) < 1e-14
    dz = np.concatenate([ox.vocab_parallel_xent_bwd(s, y, a, gmax, sexp, dl) for s, a in zip(sh, v0)], 1)
    ref = np.full((N, V), 1.0 / V)
    ref[np.arange(N), y] -= 1
    assert np.max(np.abs(dz - ref * 0.5)) < 1e-15


def test_brute_force_tiny():
    z = [[0.1, -2.0, 3.5, 0.0], [1.0, 1.0, -1.0, 2.0]]
    y = [2, 1]
    zz = np.array(z)
    sh, v0 = _shards(zz, 2)
    loss, _, _ = ox.vocab_parallel_xent(sh, np.array(y), v0)
    for n in range(2):
        ref = math.log(sum(math.exp(v) for v in z[n])) - z[n][y[n]]
        assert abs(loss[n] - ref) < 1e-14
