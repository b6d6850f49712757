"""Pins for the fp64 block oracle (CPU only).

Each test checks the oracle against something other than itself: central
finite differences, the tensor-parallel shard-sum identities the pages state,
brute-force loops on tiny inputs, closed forms, a textbook normal-CDF table,
and an independent float64 autograd implementation (torch on the CPU).
"""
import math
import os

import numpy as np
import pytest

from oracle import block as ob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_weights(rng, H, nq, nkv, d, F, act, bias, affine):
    s = 1.0 / math.sqrt(H)
    w = {"wq": rng.normal(0, s, (nq * d, H)), "wk": rng.normal(0, s, (nkv * d, H)),
         "wv": rng.normal(0, s, (nkv * d, H)), "wo": rng.normal(0, 1 / math.sqrt(nq * d), (H, nq * d)),
         "w2": rng.normal(0, 1 / math.sqrt(F), (H, F))}
    if act == "gelu":
        w["w1"] = rng.normal(0, s, (F, H))
    else:
        w["wg"] = rng.normal(0, s, (F, H))
        w["wu"] = rng.normal(0, s, (F, H))
    if bias:
        for k, n in (("bq", nq * d), ("bk", nkv * d), ("bv", nkv * d), ("bo", H), ("b2", H)):
            w[k] = rng.normal(0, 0.3, n)
        for k in (("b1",) if act == "gelu" else ("bg", "bu")):
            w[k] = rng.normal(0, 0.3, F)
    if affine:
        for k in ("ln1_g", "ln2_g"):
            w[k] = 1 + 0.2 * rng.normal(size=H)
        for k in ("ln1_b", "ln2_b"):
            w[k] = 0.2 * rng.normal(size=H)
    return w


VARIANTS = [
    # act, causal, bias, affine, nq, nkv, R, norm
    ("gelu", False, False, False, 2, 2, 1, "pre"),
    ("gelu", True, True, True, 2, 2, 2, "pre"),
    ("swiglu", True, True, True, 4, 2, 2, "pre"),    # GQA: 2 q heads per kv head
    ("swiglu", False, False, False, 4, 1, 1, "pre"),  # MQA-like: 4 q heads share 1 kv head
    ("gelu", True, True, True, 2, 2, 2, "post"),      # post-LN ([Lab06] sec. 2 (2)(5))
    ("swiglu", False, False, False, 4, 2, 1, "post"),
]


def _fwd(x, w, v, R=None):
    act, causal, _, _, nq, nkv, r, norm = v
    return ob.block_forward(x, w, q_heads=nq, kv_heads=nkv, head_dim=4, act=act,
                            causal=causal, R=r if R is None else R, norm=norm)


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: f"{v[0]}-c{int(v[1])}-b{int(v[2])}-a{int(v[3])}-q{v[4]}kv{v[5]}-R{v[6]}-{v[7]}")
def test_block_backward_matches_central_differences(v):
    """Every gradient (dx and all weights) against central differences of
    L = sum(out * G), step 1e-6, on B=2, S=5, H=8, d=4, F=6."""
    act, causal, bias, affine, nq, nkv, R, _ = v
    rng = np.random.default_rng(7)
    B, S, H, d, F = 2, 5, 8, 4, 6
    x = rng.normal(size=(B, S, H))
    G = rng.normal(size=(B, S, H))
    w = _rand_weights(rng, H, nq, nkv, d, F, act, bias, affine)
    out, cache = _fwd(x, w, v)
    dx, grads = ob.block_backward(G, cache)

    def L(xx, ww):
        o, _ = _fwd(xx, ww, v)
        return float((o * G).sum())

    h = 1e-6
    # dx
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy(); xp[idx] += h
        xm = x.copy(); xm[idx] -= h
        fd[idx] = (L(xp, w) - L(xm, w)) / (2 * h)
    assert np.max(np.abs(fd - dx)) <= 1e-6 * max(1.0, np.max(np.abs(dx)))
    # every weight
    for k in w:
        fdk = np.zeros_like(w[k])
        for idx in np.ndindex(*w[k].shape):
            wp = dict(w); wp[k] = w[k].copy(); wp[k][idx] += h
            wm = dict(w); wm[k] = w[k].copy(); wm[k][idx] -= h
            fdk[idx] = (L(x, wp) - L(x, wm)) / (2 * h)
        err = np.max(np.abs(fdk - grads[k]))
        assert err <= 1e-6 * max(1.0, np.max(np.abs(grads[k]))), (k, err)


@pytest.mark.parametrize("norm", ["pre", "post"])
def test_shard_sum_identity_forward_and_backward(norm):
    """Splitting the layer over R = 4 ranks (whole heads, ffn/R columns) and
    summing the row-parallel partials reproduces the unsharded block, its
    input gradient and every weight gradient ([TP-block] sec. 1-2)."""
    rng = np.random.default_rng(11)
    B, S, H, nq, nkv, d, F = 2, 8, 16, 4, 4, 4, 8
    for act in ("gelu", "swiglu"):
        w = _rand_weights(rng, H, nq, nkv, d, F, act, True, True)
        x = rng.normal(size=(B, S, H))
        G = rng.normal(size=(B, S, H))
        kw = dict(q_heads=nq, kv_heads=nkv, head_dim=d, act=act, causal=True, norm=norm)
        o1, c1 = ob.block_forward(x, w, R=1, **kw)
        o4, c4 = ob.block_forward(x, w, R=4, **kw)
        dx1, g1 = ob.block_backward(G, c1)
        dx4, g4 = ob.block_backward(G, c4)
        rel = lambda a, b: np.max(np.abs(a - b)) / max(1.0, np.max(np.abs(b)))
        assert rel(o4, o1) < 1e-12
        assert rel(dx4, dx1) < 1e-12
        for k in w:
            assert rel(g4[k], g1[k]) < 1e-12, k
        # a key bias shifts every score of a row by the same amount, which
        # softmax ignores: its gradient is exactly zero
        assert np.max(np.abs(g1["bk"])) < 1e-13
        # the partials really are partial: no single shard equals the sum
        assert rel(c4["p_attn"][0], c1["p_attn"][0]) > 1e-3
        assert rel(sum(c4["p_attn"]), c1["p_attn"][0]) < 1e-12
        assert rel(sum(g4["_dc_partials"]), g1["_dc_partials"][0]) < 1e-12
        assert rel(sum(g4["_da_partials"]), g1["_da_partials"][0]) < 1e-12
        # column-parallel outputs concatenate with no reduction
        q1 = c1["shards"][0]["q"]
        q4 = np.concatenate([c4["shards"][r]["q"] for r in range(4)], axis=1)
        assert rel(q4, q1) < 1e-14


def test_softmax_rows_sum_to_one_and_causal_zeros():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(9, 8)) * 3
    k = rng.normal(size=(9, 8)) * 3
    for causal in (False, True):
        p = ob.attention_probs(q, k, causal)
        assert np.max(np.abs(p.sum(-1) - 1)) < 1e-12
        assert np.all(p >= 0)
        if causal:
            assert np.all(p[np.triu_indices(9, 1)] == 0.0)
            assert p[0, 0] == 1.0


def test_attention_brute_force_tiny():
    """Pure-Python triple loops with math.exp on S=3, d=2, two q heads
    sharing one kv head."""
    rng = np.random.default_rng(5)
    q = rng.normal(size=(1, 2, 3, 2))
    k = rng.normal(size=(1, 1, 3, 2))
    v = rng.normal(size=(1, 1, 3, 2))
    for causal in (False, True):
        o = ob.attention_fwd(q, k, v, causal)
        for i in range(2):
            for s in range(3):
                keys = range(s + 1) if causal else range(3)
                sc = [sum(q[0, i, s, e] * k[0, 0, t, e] for e in range(2)) / math.sqrt(2) for t in keys]
                mx = max(sc)
                ex = [math.exp(z - mx) for z in sc]
                tot = sum(ex)
                for e in range(2):
                    ref = sum(ex[j] / tot * v[0, 0, t, e] for j, t in enumerate(keys))
                    assert abs(o[0, i, s, e] - ref) < 1e-14


def test_layernorm_brute_force_and_moments():
    rng = np.random.default_rng(9)
    x = rng.normal(size=(4, 7)) * 5 + 2
    y, xhat, rstd = ob.layer_norm_fwd(x, eps=1e-5)
    for t in range(4):
        row = list(x[t])
        mu = sum(row) / 7
        var = sum((r - mu) ** 2 for r in row) / 7
        for h in range(7):
            assert abs(y[t, h] - (row[h] - mu) / math.sqrt(var + 1e-5)) < 1e-13
        # output rows: mean 0 and biased variance var/(var+eps)
        assert abs(y[t].mean()) < 1e-14
        assert abs(y[t].var() - var / (var + 1e-5)) < 1e-13


def test_gelu_against_normal_table():
    tab = np.loadtxt(os.path.join(GOLDEN, "normal_cdf_table.txt"))
    u, cdf, pdf = tab[:, 0], tab[:, 1], tab[:, 2]
    assert np.max(np.abs(ob.gelu(u) - u * cdf)) < 1e-15
    assert np.max(np.abs(ob.gelu_grad(u) - (cdf + u * pdf))) < 1e-15
    assert ob.gelu(np.array(0.0)) == 0.0 and ob.gelu_grad(np.array(0.0)) == 0.5


def test_closed_forms_single_token_and_zero_projections():
    rng = np.random.default_rng(13)
    H, nq, nkv, d, F = 8, 2, 1, 4, 6
    w = _rand_weights(rng, H, nq, nkv, d, F, "gelu", False, False)
    # S = 1: softmax over one key is 1, so each q head's output is its V row
    x = rng.normal(size=(3, 1, H))
    _, c = ob.block_forward(x, w, q_heads=nq, kv_heads=nkv, head_dim=d, causal=False)
    sh = c["shards"][0]
    v = c["a"] @ w["wv"].T
    for i in range(nq):
        assert np.max(np.abs(sh["o"][:, i * d:(i + 1) * d] - v)) < 1e-14
    # zero output projections: out = x and dx = G
    w0 = dict(w)
    w0["wo"] = np.zeros_like(w["wo"])
    w0["w2"] = np.zeros_like(w["w2"])
    x = rng.normal(size=(2, 5, H))
    G = rng.normal(size=(2, 5, H))
    out, c = ob.block_forward(x, w0, q_heads=nq, kv_heads=nkv, head_dim=d, causal=True)
    dx, _ = ob.block_backward(G, c)
    assert np.array_equal(out, x)
    assert np.max(np.abs(dx - G)) < 1e-15


def test_identical_keys_give_prefix_means():
    """All keys equal -> uniform weights over the visible keys -> O is the
    mean of V over those keys (prefix means when causal)."""
    rng = np.random.default_rng(17)
    S, d = 6, 4
    q = rng.normal(size=(1, 1, S, d))
    k = np.tile(rng.normal(size=(1, 1, 1, d)), (1, 1, S, 1))
    v = rng.normal(size=(1, 1, S, d))
    o = ob.attention_fwd(q, k, v, False)
    assert np.max(np.abs(o[0, 0] - v[0, 0].mean(0))) < 1e-14
    o = ob.attention_fwd(q, k, v, True)
    pref = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    assert np.max(np.abs(o[0, 0] - pref)) < 1e-14


@pytest.mark.parametrize("norm", ["pre", "post"])
def test_against_independent_float64_autograd(norm):
    """The same block written with torch float64 CPU ops and autograd
    (post-LN: LN(x + attention(x)), then LN(h + MLP(h)))."""
    torch = pytest.importorskip("torch")
    F_ = torch.nn.functional
    rng = np.random.default_rng(21)
    B, S, H, nq, nkv, d, F = 2, 7, 16, 4, 2, 4, 12
    post = norm == "post"
    for act, causal in (("gelu", False), ("swiglu", True)):
        w = _rand_weights(rng, H, nq, nkv, d, F, act, True, True)
        x = rng.normal(size=(B, S, H))
        G = rng.normal(size=(B, S, H))
        out, c = ob.block_forward(x, w, q_heads=nq, kv_heads=nkv, head_dim=d, act=act, causal=causal,
                                  norm=norm)
        dx, grads = ob.block_backward(G, c)

        tw = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in w.items()}
        tx = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        a = tx if post else F_.layer_norm(tx, (H,), tw["ln1_g"], tw["ln1_b"], 1e-5)
        q = F_.linear(a, tw["wq"], tw["bq"]).view(B, S, nq, d).permute(0, 2, 1, 3)
        k = F_.linear(a, tw["wk"], tw["bk"]).view(B, S, nkv, d).permute(0, 2, 1, 3)
        v = F_.linear(a, tw["wv"], tw["bv"]).view(B, S, nkv, d).permute(0, 2, 1, 3)
        k = k.repeat_interleave(nq // nkv, dim=1)
        v = v.repeat_interleave(nq // nkv, dim=1)
        sc = torch.matmul(q, k.transpose(-1, -2)) / d ** 0.5
        if causal:
            sc = sc.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
        o = torch.matmul(torch.softmax(sc, -1), v).permute(0, 2, 1, 3).reshape(B, S, nq * d)
        hh = tx + F_.linear(o, tw["wo"], tw["bo"])
        if post:
            hh = F_.layer_norm(hh, (H,), tw["ln1_g"], tw["ln1_b"], 1e-5)
            cc = hh
        else:
            cc = F_.layer_norm(hh, (H,), tw["ln2_g"], tw["ln2_b"], 1e-5)
        if act == "gelu":
            m = F_.gelu(F_.linear(cc, tw["w1"], tw["b1"]))
        else:
            m = F_.silu(F_.linear(cc, tw["wg"], tw["bg"])) * F_.linear(cc, tw["wu"], tw["bu"])
        to = hh + F_.linear(m, tw["w2"], tw["b2"])
        if post:
            to = F_.layer_norm(to, (H,), tw["ln2_g"], tw["ln2_b"], 1e-5)
        (to * torch.tensor(G)).sum().backward()
        assert np.max(np.abs(to.detach().numpy() - out)) < 1e-12
        assert np.max(np.abs(tx.grad.numpy() - dx)) < 1e-11
        for kk in w:
            assert np.max(np.abs(tw[kk].grad.numpy() - grads[kk])) < 1e-11, kk


def test_mean_loss_cotangent_leaves_layernorm_grad_zero_without_affine():
    """Why parity also uses a random cotangent: with loss = mean(out) the
    upstream gradient is constant along each row, and LayerNorm without a
    gain maps a row-constant gradient to exactly zero."""
    rng = np.random.default_rng(23)
    x = rng.normal(size=(3, 10))
    _, xhat, rstd = ob.layer_norm_fwd(x)
    dx, _, _ = ob.layer_norm_bwd(np.full((3, 10), 0.01), xhat, rstd)
    assert np.max(np.abs(dx)) < 1e-15


def test_mean_loss_value_and_gradient():
    """block_loss_mean against what fixes it without retyping it: a brute
    force Python sum over the elements divided by their count, the mean of a
    constant tensor (that constant), and a central difference of the loss in
    a few positions (the gradient 1/numel, the same everywhere)."""
    rng = np.random.default_rng(31)
    out = rng.normal(size=(2, 3, 5))
    loss, g = ob.block_loss_mean(out)
    total, count = 0.0, 0
    for v in out.ravel().tolist():
        total += v
        count += 1
    assert abs(loss - total / count) < 1e-14
    assert abs(ob.block_loss_mean(np.full((4, 7), 2.5))[0] - 2.5) < 1e-15
    assert g.shape == out.shape
    h = 1e-6
    for idx in [(0, 0, 0), (1, 2, 4), (0, 1, 3)]:
        e = np.zeros_like(out)
        e[idx] = h
        fd = (ob.block_loss_mean(out + e)[0] - ob.block_loss_mean(out - e)[0]) / (2 * h)
        assert abs(fd - g[idx]) < 1e-8 and abs(g[idx] - 1.0 / 30) < 1e-15


def test_post_ln_closed_form_with_zero_projections():
    """Post-LN with Wo = W2 = 0 and no biases: out = LN(LN(x)) row by row.
    Written out: y = (x - mean) / sqrt(var + eps) has variance
    var / (var + eps), so out = y / sqrt(var / (var + eps) + eps). Its input
    gradient (through two gain-free LayerNorms) has zero row sums."""
    rng = np.random.default_rng(29)
    H, nq, nkv, d, F = 12, 2, 2, 4, 8
    w = _rand_weights(rng, H, nq, nkv, d, F, "gelu", False, False)
    w["wo"] = np.zeros_like(w["wo"])
    w["w2"] = np.zeros_like(w["w2"])
    x = rng.normal(size=(2, 5, H)) * 3.0 + 1.0
    G = rng.normal(size=(2, 5, H))
    out, c = ob.block_forward(x, w, q_heads=nq, kv_heads=nkv, head_dim=d, causal=True, norm="post")
    eps = 1e-5
    mu = x.mean(-1, keepdims=True)
    var = x.var(-1, keepdims=True)
    ref = (x - mu) / np.sqrt(var + eps) / np.sqrt(var / (var + eps) + eps)
    assert np.max(np.abs(out - ref)) < 1e-13
    dx, _ = ob.block_backward(G, c)
    assert np.max(np.abs(dx.sum(-1))) < 1e-13


def test_post_ln_output_rows_are_normalised():
    """Whatever the weights, a gain-free post-LN block's output rows have
    mean 0 and variance v / (v + eps) (v: the row variance of r2 = h + mlp),
    so strictly inside (0, 1) and close to 1 for unit-scale rows."""
    rng = np.random.default_rng(31)
    H, nq, nkv, d, F = 16, 4, 2, 4, 12
    for act in ("gelu", "swiglu"):
        w = _rand_weights(rng, H, nq, nkv, d, F, act, True, False)
        x = rng.normal(size=(2, 6, H))
        out, c = ob.block_forward(x, w, q_heads=nq, kv_heads=nkv, head_dim=d, act=act, norm="post")
        assert np.max(np.abs(out.mean(-1))) < 1e-14
        v = out.var(-1)
        assert np.all(v < 1.0) and np.all(v > 0.999)
        # and the MLP read the first LayerNorm's output, itself normalised
        assert np.max(np.abs(c["c"].mean(-1))) < 1e-14
