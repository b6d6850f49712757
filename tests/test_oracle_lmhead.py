"""Pins of the LM head + vocab-parallel cross-entropy oracle: central finite
differences of the weighted loss, the sharded result against the unsharded
one, and an independent float64 autograd of torch's cross_entropy."""
import numpy as np
import pytest

from oracle import lmhead as ol
from oracle import xent as ox


def _case(n=5, H=6, V=12, R=3, seed=0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((n, H))
    w = rng.standard_normal((V, H)) * 0.7
    target = rng.integers(0, V, size=n)
    dloss = rng.uniform(0.5, 1.5, size=n)
    ranges = ox.shard_ranges(V, R)
    return h, w, target, dloss, [w[a:b] for a, b in ranges], [a for a, _ in ranges]


def _grads(h, w, target, dloss, R):
    ranges = ox.shard_ranges(w.shape[0], R)
    ws = [w[a:b] for a, b in ranges]
    starts = [a for a, _ in ranges]
    loss, gmax, se, zs = ol.forward(h, ws, target, starts)
    dh = np.zeros_like(h)
    dws = []
    for wr, zr, v0 in zip(ws, zs, starts):
        a, b = ol.backward_shard(h, wr, zr, target, v0, gmax, se, dloss)
        dh += a
        dws.append(b)
    return loss, dh, np.concatenate(dws)


def test_finite_differences_of_the_weighted_loss():
    h, w, target, dloss, _, _ = _case()
    _, dh, dw = _grads(h, w, target, dloss, R=3)
    f = lambda hh, ww: float(np.sum(dloss * _grads(hh, ww, target, dloss, R=3)[0]))
    eps = 1e-6
    for (i, j) in [(0, 0), (2, 3), (4, 5)]:
        hp, hm = h.copy(), h.copy()
        hp[i, j] += eps
        hm[i, j] -= eps
        assert abs((f(hp, w) - f(hm, w)) / (2 * eps) - dh[i, j]) <= 1e-6 * max(1.0, abs(dh[i, j]))
    for (i, j) in [(0, 1), (5, 2), (11, 5)]:
        wp, wm = w.copy(), w.copy()
        wp[i, j] += eps
        wm[i, j] -= eps
        assert abs((f(h, wp) - f(h, wm)) / (2 * eps) - dw[i, j]) <= 1e-6 * max(1.0, abs(dw[i, j]))


@pytest.mark.parametrize("R", [2, 3, 6])
def test_sharded_equals_unsharded(R):
    h, w, target, dloss, _, _ = _case(n=7, V=12, seed=2)
    l1, dh1, dw1 = _grads(h, w, target, dloss, R=1)
    lr, dhr, dwr = _grads(h, w, target, dloss, R=R)
    np.testing.assert_allclose(lr, l1, rtol=1e-12, atol=0)
    np.testing.assert_allclose(dhr, dh1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dwr, dw1, rtol=0, atol=1e-12)


def test_matches_float64_autograd_cross_entropy():
    torch = pytest.importorskip("torch")
    h, w, target, dloss, _, _ = _case(n=9, H=5, V=15, seed=4)
    loss, dh, dw = _grads(h, w, target, dloss, R=5)
    th = torch.tensor(h, dtype=torch.float64, requires_grad=True)
    tw = torch.tensor(w, dtype=torch.float64, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(th @ tw.T, torch.tensor(target), reduction="none")
    (tl * torch.tensor(dloss)).sum().backward()
    np.testing.assert_allclose(loss, tl.detach().numpy(), rtol=1e-12, atol=0)
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=0, atol=1e-12)
