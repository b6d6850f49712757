"""Pins for the oracle's counter-based dropout ([TP-block] sec. 5) and for the
block with dropout (CPU only).

The generator is pinned to the known-answer vectors published with the
Philox4x32-10 reference implementation (Salmon et al., SC 2011, "Parallel
random numbers: as easy as 1, 2, 3"); the masks to their statistics and to
the counter semantics; the block with dropout to central differences (the
masks are a pure function of the seed, so the block stays a deterministic
function of its inputs), to a float64 torch autograd of the masked block, and
to the no-dropout block at p = 0.
"""
import math

import numpy as np
import pytest

from oracle import block as ob
from oracle import dropout as od

from test_oracle_block import _rand_weights


# (counter words, key words) -> output words
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("c,k,ref", KAT)
def test_philox_known_answers(c, k, ref):
    out = od.philox4x32_10(*c, *k)
    assert tuple(int(v) for v in out) == ref


def test_philox_vectorised_equals_scalar():
    rng = np.random.default_rng(3)
    c = rng.integers(0, 2 ** 32, size=(4, 50), dtype=np.uint64)
    k = (0x12345678, 0x9abcdef0)
    vec = od.philox4x32_10(c[0], c[1], c[2], c[3], *k)
    for j in range(50):
        one = od.philox4x32_10(c[0, j], c[1, j], c[2, j], c[3, j], *k)
        assert all(int(vec[w][j]) == int(one[w]) for w in range(4))


def test_threshold_is_the_integer_floor():
    assert od.threshold(0.0) == 0
    assert od.threshold(0.5) == 2 ** 31
    assert od.threshold(0.25) == 2 ** 30
    assert od.threshold(0.1) == math.floor(0.1 * 2 ** 32)
    assert od.threshold(1.0 - 2 ** -40) == 2 ** 32 - 1
    with pytest.raises(ValueError):
        od.threshold(1.0)


def test_words_are_uniform_and_masks_drop_p():
    n = 1 << 20
    w = od.words(np.arange(n, dtype=np.uint64), od.SITE_HIDDEN_MLP, 1234, 7).astype(np.float64)
    u = w / 2 ** 32
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / n)
    counts = np.bincount((u * 16).astype(np.int64), minlength=16)
    chi2 = ((counts - n / 16) ** 2 / (n / 16)).sum()
    assert chi2 < 60          # 15 degrees of freedom: p-value ~1e-7 at 60
    for p in (0.1, 0.5, 0.9):
        keep = od.keep_mask((n,), od.SITE_ATTN, 99, 0, p)
        drop = 1.0 - keep.mean()
        assert abs(drop - p) < 5 * math.sqrt(p * (1 - p) / n), (p, drop)
        m = od.multiplier((n,), od.SITE_ATTN, 99, 0, p)
        assert abs(m.mean() - 1.0) < 5 * math.sqrt(p / (1 - p) / n)


def test_mask_is_a_function_of_the_element_index():
    """Any subset of indices gets the same words as the whole range (what
    lets every kernel compute only its own elements), and (seed, site,
    offset) each select a different stream."""
    n = 4096
    full = od.words(np.arange(n, dtype=np.uint64), 1, 55, 3)
    idx = np.array([5, 4095, 0, 1, 2, 3, 1000, 2049], dtype=np.uint64)
    assert np.array_equal(od.words(idx, 1, 55, 3), full[idx.astype(np.int64)])
    # high counter word: index 2^34 + i differs from i
    big = od.words(np.arange(n, dtype=np.uint64) + np.uint64(1 << 34), 1, 55, 3)
    assert (big != full).mean() > 0.99
    for other in (od.words(np.arange(n, dtype=np.uint64), 2, 55, 3),
                  od.words(np.arange(n, dtype=np.uint64), 1, 56, 3),
                  od.words(np.arange(n, dtype=np.uint64), 1, 55, 4),
                  od.words(np.arange(n, dtype=np.uint64), 1, 55 + (1 << 32), 3)):
        assert (other != full).mean() > 0.99


DROP = dict(p_attn=0.3, p_hidden=0.2, seed=20240917, offset=5)


def _kw(nq, nkv, act, causal, norm, d=4):
    return dict(q_heads=nq, kv_heads=nkv, head_dim=d, act=act, causal=causal, norm=norm)


def test_zero_probabilities_give_the_plain_block():
    rng = np.random.default_rng(41)
    H, nq, nkv, d, F = 16, 4, 2, 4, 12
    w = _rand_weights(rng, H, nq, nkv, d, F, "swiglu", True, True)
    x = rng.normal(size=(2, 6, H))
    G = rng.normal(size=(2, 6, H))
    for norm in ("pre", "post"):
        kw = _kw(nq, nkv, "swiglu", True, norm)
        o0, c0 = ob.block_forward(x, w, **kw)
        o1, c1 = ob.block_forward(x, w, dropout=dict(DROP, p_attn=0.0, p_hidden=0.0), **kw)
        assert np.array_equal(o0, o1)
        dx0, g0 = ob.block_backward(G, c0)
        dx1, g1 = ob.block_backward(G, c1)
        assert np.array_equal(dx0, dx1)
        for k in w:
            assert np.array_equal(g0[k], g1[k])
        o2, _ = ob.block_forward(x, w, dropout=DROP, **kw)
        assert np.max(np.abs(o2 - o0)) > 0.1


def test_tensor_parallel_seeds():
    """[TP-block] sec. 5: the hidden masks (outside the TP region) are the
    same on every rank; the attention masks (inside) differ per rank; and
    the R-shard block equals R single-rank blocks run with tp_rank = r."""
    rng = np.random.default_rng(43)
    H, nq, nkv, d, F, R = 16, 4, 4, 4, 8, 2
    w = _rand_weights(rng, H, nq, nkv, d, F, "gelu", False, False)
    x = rng.normal(size=(1, 8, H))
    kw = _kw(nq, nkv, "gelu", False, "pre")
    _, c = ob.block_forward(x, w, R=R, dropout=DROP, **kw)
    m0, m1 = np.asarray(c["shards"][0]["mult"]), np.asarray(c["shards"][1]["mult"])
    assert m0.shape == m1.shape and (m0 != m1).mean() > 0.3
    # rank 1 of two = shard 0 of a one-shard run at tp_rank 1
    _, c1 = ob.block_forward(x, ob.shard(w, R, 1, d), R=1, dropout=DROP, tp_rank=1,
                             **dict(kw, q_heads=nq // R, kv_heads=nkv // R))
    assert np.array_equal(np.asarray(c1["shards"][0]["mult"]), m1)
    # the per-(batch, head) slices are the full-array mask's slices
    full = od.keep_mask((1, nq // R, 8, 8), od.SITE_ATTN, od.attn_seed(DROP["seed"], 1),
                        DROP["offset"], DROP["p_attn"]) / (1 - DROP["p_attn"])
    assert np.array_equal(full, m1)
    _, c0 = ob.block_forward(x, ob.shard(w, R, 0, d), R=1, dropout=DROP, tp_rank=0,
                             **dict(kw, q_heads=nq // R, kv_heads=nkv // R))
    assert np.array_equal(c0["mult_h1"], c1["mult_h1"]) and np.array_equal(c0["mult_h2"], c1["mult_h2"])
    assert np.array_equal(c0["mult_h1"], c["mult_h1"])
    assert (c["mult_h1"] != c["mult_h2"]).mean() > 0.1


@pytest.mark.parametrize("norm,act,causal", [("pre", "gelu", True), ("post", "swiglu", False)])
def test_dropout_block_backward_matches_central_differences(norm, act, causal):
    rng = np.random.default_rng(47)
    B, S, H, nq, nkv, d, F = 2, 5, 8, 2, 1, 4, 6
    x = rng.normal(size=(B, S, H))
    G = rng.normal(size=(B, S, H))
    w = _rand_weights(rng, H, nq, nkv, d, F, act, True, True)
    kw = dict(_kw(nq, nkv, act, causal, norm), dropout=DROP)
    out, cache = ob.block_forward(x, w, **kw)
    dx, grads = ob.block_backward(G, cache)

    def L(xx, ww):
        o, _ = ob.block_forward(xx, ww, **kw)
        return float((o * G).sum())

    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        fd[idx] = (L(xp, w) - L(xm, w)) / (2 * h)
    assert np.max(np.abs(fd - dx)) <= 1e-6 * max(1.0, np.max(np.abs(dx)))
    for k in ("wq", "wo", "w2", "bo", "b2", "ln1_g", "ln2_b"):
        fdk = np.zeros_like(w[k])
        for idx in np.ndindex(*w[k].shape):
            wp = dict(w); wp[k] = w[k].copy(); wp[k][idx] += h
            wm = dict(w); wm[k] = w[k].copy(); wm[k][idx] -= h
            fdk[idx] = (L(x, wp) - L(x, wm)) / (2 * h)
        err = np.max(np.abs(fdk - grads[k]))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(grads[k]))), (k, err)


def test_masked_block_against_float64_autograd():
    """The pre-LN block with the oracle's masks applied by torch float64 ops
    (P * mult before P V, hidden multipliers before each residual add)."""
    torch = pytest.importorskip("torch")
    F_ = torch.nn.functional
    rng = np.random.default_rng(53)
    B, S, H, nq, nkv, d, F = 2, 7, 16, 4, 2, 4, 12
    w = _rand_weights(rng, H, nq, nkv, d, F, "gelu", True, True)
    x = rng.normal(size=(B, S, H))
    G = rng.normal(size=(B, S, H))
    out, c = ob.block_forward(x, w, dropout=DROP, **_kw(nq, nkv, "gelu", True, "pre"))
    dx, grads = ob.block_backward(G, c)
    T = B * S
    tw = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in w.items()}
    tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    a = F_.layer_norm(tx, (H,), tw["ln1_g"], tw["ln1_b"], 1e-5)
    q = F_.linear(a, tw["wq"], tw["bq"]).view(B, S, nq, d).permute(0, 2, 1, 3)
    k = F_.linear(a, tw["wk"], tw["bk"]).view(B, S, nkv, d).permute(0, 2, 1, 3)
    v = F_.linear(a, tw["wv"], tw["bv"]).view(B, S, nkv, d).permute(0, 2, 1, 3)
    k = k.repeat_interleave(nq // nkv, dim=1)
    v = v.repeat_interleave(nq // nkv, dim=1)
    sc = torch.matmul(q, k.transpose(-1, -2)) / d ** 0.5
    sc = sc.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    pm = torch.softmax(sc, -1) * torch.tensor(np.asarray(c["shards"][0]["mult"]))
    o = torch.matmul(pm, v).permute(0, 2, 1, 3).reshape(B, S, nq * d)
    m1 = torch.tensor(c["mult_h1"].reshape(B, S, H))
    m2 = torch.tensor(c["mult_h2"].reshape(B, S, H))
    hh = tx + F_.linear(o, tw["wo"], tw["bo"]) * m1
    cc = F_.layer_norm(hh, (H,), tw["ln2_g"], tw["ln2_b"], 1e-5)
    to = hh + F_.linear(F_.gelu(F_.linear(cc, tw["w1"], tw["b1"])), tw["w2"], tw["b2"]) * m2
    (to * torch.tensor(G)).sum().backward()
    assert np.max(np.abs(to.detach().numpy() - out)) < 1e-12
    assert np.max(np.abs(tx.grad.numpy() - dx)) < 1e-11
    for kk in w:
        assert np.max(np.abs(tw[kk].grad.numpy() - grads[kk])) < 1e-11, kk
    assert T == out.reshape(-1, H).shape[0]
