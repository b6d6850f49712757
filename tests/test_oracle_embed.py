"""Pins of the vocab-parallel embedding oracle ([TP-block] sec. 3) against
facts fixed by the definition, not by the oracle's own code: a full-table
lookup (numpy fancy indexing on the unsplit table), the adjoint identity of a
linear map, a dense one-hot product, brute-force loops, special cases."""
import numpy as np
import pytest

from oracle import embed as oe


def _case(n=37, vocab=48, h=8, R=4, seed=0, ids=None):
    rng = np.random.default_rng(seed)
    table = rng.standard_normal((vocab, h))
    if ids is None:
        ids = rng.integers(0, vocab, size=n)
    starts = [a for a, _ in oe.shard_ranges(vocab, R)]
    tables = [table[a:b] for a, b in oe.shard_ranges(vocab, R)]
    return rng, table, np.asarray(ids, np.int64), starts, tables


@pytest.mark.parametrize("R", [1, 2, 4, 8])
def test_shard_sum_equals_full_table_lookup(R):
    _, table, ids, starts, tables = _case(vocab=64, R=R)
    out = oe.embed_fwd_sharded(tables, ids, starts)
    assert np.array_equal(out, table[ids])          # exactly one non-zero term per token


def test_each_token_owned_by_exactly_one_shard():
    _, table, ids, starts, tables = _case(R=4)
    nonzero = np.stack([np.abs(oe.embed_fwd(t, ids, v0)).sum(1) > 0 for t, v0 in zip(tables, starts)])
    assert np.array_equal(nonzero.sum(0), np.ones(len(ids)))


def test_ids_outside_the_shard_give_zero_rows():
    _, table, _, starts, tables = _case(R=4)
    ids = np.array([-5, 12, 11, 0, 47, 48, 1000], np.int64)   # shard 1 holds [12, 24)
    out = oe.embed_fwd(tables[1], ids, starts[1])
    assert np.array_equal(out[1], table[12])
    for t in (0, 2, 3, 4, 5, 6):
        assert not out[t].any()


@pytest.mark.parametrize("R", [1, 4])
def test_backward_is_the_adjoint_of_the_forward(R):
    rng, table, ids, starts, tables = _case(n=53, vocab=32, R=R, seed=3)
    G = rng.standard_normal((len(ids), table.shape[1]))
    for t, v0 in zip(tables, starts):
        lhs = float(np.sum(oe.embed_fwd(t, ids, v0) * G))
        rhs = float(np.sum(t * oe.embed_bwd(G, ids, v0, t.shape[0])))
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_backward_equals_dense_one_hot_product():
    rng, table, ids, starts, tables = _case(n=70, vocab=40, R=2, seed=5)
    G = rng.standard_normal((len(ids), table.shape[1]))
    onehot = np.zeros((len(ids), table.shape[0]))
    onehot[np.arange(len(ids)), ids] = 1.0
    full = onehot.T @ G                               # d(table) of out = onehot @ table
    parts = [oe.embed_bwd(G, ids, v0, t.shape[0]) for t, v0 in zip(tables, starts)]
    np.testing.assert_allclose(np.concatenate(parts), full, rtol=0, atol=1e-12)


def test_backward_brute_force_tiny():
    G = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    ids = np.array([2, 0, 2, 5], np.int64)           # shard [0, 3): rows 0 and 2 hit
    d = oe.embed_bwd(G, ids, 0, 3)
    assert np.array_equal(d, np.array([[3.0, 4.0], [0.0, 0.0], [1.0 + 5.0, 2.0 + 6.0]]))


def test_backward_each_id_once_is_a_row_permutation():
    rng = np.random.default_rng(9)
    ids = rng.permutation(16).astype(np.int64)
    G = rng.standard_normal((16, 4))
    d = oe.embed_bwd(G, ids, 0, 16)
    assert np.array_equal(d[ids], G)
