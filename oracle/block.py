"""fp64 oracle of one Megatron-style tensor-parallel Transformer block,
forward and backward (test infrastructure only; see the package docstring).

Structure ([Lab06] sec. 2 listing, steps (2)-(8); [TP-block] sec. 1-2):

    a   = LN1(x)                                   (2)
    qkv = a Wqkv^T + bqkv      column-parallel, split by head
    O   = softmax(Q K^T / sqrt(d)) V per head      (attention over the sequence)
    attn= sum_r O_r Wo_r^T + bo  row-parallel partials, reduction point g1
    h   = x + attn                                  (4)
    c   = LN2(h)                                    (5)
    m   = GELU(c W1^T + b1)  or  silu(c Wg^T + bg) * (c Wu^T + bu)
    out = h + sum_r m_r W2_r^T + b2   row-parallel partials, reduction point g2  (6)(7)

Post-LN variant ([Lab06] sec. 2 notes (2)(5) and sec. 5: the residual is
added first and the sum is normalised, as in the original Transformer):

    r1  = x + attn(x)          h   = LN1(r1)
    r2  = h + mlp(h)           out = LN2(r2)

with the same attention and MLP (and the same reduction points); the
attention reads x itself and the MLP reads h.

Dropout ([TP-block] sec. 5), optional: on the attention probabilities of each
local head (inside the TP region: rank r draws with seed + 2718 + r), and on
the hidden state after the attention block and after the MLP, i.e. on
sum(partials) + bias before the residual add (outside the TP region: every
rank draws the same mask from the seed itself). Masks come from the
counter-based generator in ``dropout``; a kept value is scaled by 1/(1-p).

The backward follows the conjugate placement of the reductions: a
row-parallel output is summed in the forward and passed through in the
backward; a column-parallel input is passed through in the forward and its
gradient is summed over shards in the backward ([TP-block] sec. 2: two
reductions forward, two backward).

Readings of points the pages leave open (each pinned by a test):
pre-LN order as the listing codes it (no final LN); attention per head over
the sequence axis; the attention output goes through a row-parallel
projection; LayerNorm uses the biased variance, eps = 1e-5, and an optional
gain/shift; GELU is the exact erf form; SwiGLU is silu(gate) * up; q head i
reads kv head floor(i / (nq / nkv)); packed QKV rows are [Q | K | V];
row-parallel biases are added once, after the shard sum.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf

from . import dropout as odrop

F64 = np.float64


# --------------------------------------------------------------------------
# LayerNorm ([Lab06] sec. 2 steps (2) and (5): F.layer_norm over hidden)
# --------------------------------------------------------------------------
def layer_norm_fwd(x, gamma=None, beta=None, eps=1e-5):
    """Per-row normalisation over the last axis with the biased variance.
    Returns (y, xhat, rstd)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    y = xhat
    if gamma is not None:
        y = y * gamma
    if beta is not None:
        y = y + beta
    return y, xhat, rstd[..., 0]


def layer_norm_bwd(dy, xhat, rstd, gamma=None):
    """Gradient of y = xhat*gamma + beta with respect to x, gamma and beta."""
    gh = dy if gamma is None else dy * gamma
    n = xhat.shape[-1]
    dx = rstd[..., None] * (gh - gh.sum(-1, keepdims=True) / n
                            - xhat * (gh * xhat).sum(-1, keepdims=True) / n)
    dgamma = (dy * xhat).reshape(-1, n).sum(0)
    dbeta = dy.reshape(-1, n).sum(0)
    return dx, dgamma, dbeta


# --------------------------------------------------------------------------
# activations ([Lab06] sec. 2 step (6) F.gelu; [TP-block] sec. 1 SwiGLU)
# --------------------------------------------------------------------------
def gelu(u):
    """Exact GELU: u * Phi(u), Phi the standard normal CDF."""
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


def gelu_grad(u):
    """d/du [u Phi(u)] = Phi(u) + u phi(u)."""
    cdf = 0.5 * (1.0 + erf(u / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return cdf + u * pdf


def sigmoid(u):
    return 1.0 / (1.0 + np.exp(-u))


def swiglu(ug, uu):
    """silu(gate) * up."""
    return ug * sigmoid(ug) * uu


def swiglu_grad(ug, uu, dm):
    """(d gate, d up) of m = ug sigma(ug) uu."""
    s = sigmoid(ug)
    return dm * uu * s * (1.0 + ug * (1.0 - s)), dm * ug * s


# --------------------------------------------------------------------------
# attention per head ([Lab06] sec. 2 listing: scores / sqrt(head_dim),
# softmax over keys, times V; [TP-block] sec. 2 GQA)
# --------------------------------------------------------------------------
def attention_probs(qi, kj, causal):
    """P = softmax(qi kj^T / sqrt(d)) row-wise; qi [S, d], kj [S, d]."""
    d = qi.shape[-1]
    z = qi @ kj.T / math.sqrt(d)
    if causal:
        s = z.shape[0]
        z = np.where(np.triu(np.ones((s, s), dtype=bool), 1), -np.inf, z)
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=-1, keepdims=True)


def attention_fwd(q, k, v, causal, mult=None):
    """q [B, nq, S, d]; k, v [B, nkv, S, d]; q head i reads kv head i // g.
    mult [B, nq, S, S] (optional): dropout multipliers applied to P."""
    b_, nq, s, d = q.shape
    g = nq // k.shape[1]
    o = np.empty_like(q)
    for b in range(b_):
        for i in range(nq):
            p = attention_probs(q[b, i], k[b, i // g], causal)
            if mult is not None:
                p = p * mult[b, i]
            o[b, i] = p @ v[b, i // g]
    return o


def attention_bwd(q, k, v, do, causal, mult=None):
    """Gradients of O = P~ V with P~ = P o mult (mult = 1 without dropout),
    P = softmax(Z), Z = Q K^T / sqrt(d): dV += P~^T dO, dP = (dO V^T) o mult,
    dZ = P o (dP - rowsum(dP o P)), dQ = dZ K / sqrt(d), dK += dZ^T Q / sqrt(d).
    kv gradients are summed over the q heads that share the kv head."""
    b_, nq, s, d = q.shape
    g = nq // k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    sc = 1.0 / math.sqrt(d)
    for b in range(b_):
        for i in range(nq):
            j = i // g
            p = attention_probs(q[b, i], k[b, j], causal)
            pm = p if mult is None else p * mult[b, i]
            dv[b, j] += pm.T @ do[b, i]
            dp = do[b, i] @ v[b, j].T
            if mult is not None:
                dp = dp * mult[b, i]
            dz = p * (dp - (dp * p).sum(axis=-1, keepdims=True))
            dq[b, i] = dz @ k[b, j] * sc
            dk[b, j] += dz.T @ q[b, i] * sc
    return dq, dk, dv


# --------------------------------------------------------------------------
# tensor-parallel shards ([TP-block] sec. 1-2; [MLM-notes] Column/RowParallelLinear)
# --------------------------------------------------------------------------
_COL = ("wq", "wk", "wv", "w1", "wg", "wu", "bq", "bk", "bv", "b1", "bg", "bu")
_ROW = ("wo", "w2")


def shard(w, R, r, d):
    """Rank r's slice of the unsharded weights: column-parallel weights (and
    their biases) by output rows, row-parallel weights by input columns.
    Head-sized slices keep whole heads."""
    out = {}
    for k, a in w.items():
        if k in _COL:
            n = a.shape[0] // R
            out[k] = a[r * n:(r + 1) * n]
        elif k in _ROW:
            n = a.shape[1] // R
            out[k] = a[:, r * n:(r + 1) * n]
        else:
            out[k] = a
    return out


def _lin(x, w, b=None):
    y = x @ w.T
    return y if b is None else y + b


def block_forward(x, w, *, q_heads, kv_heads, head_dim, act="gelu", causal=False,
                  eps=1e-5, R=1, norm="pre", dropout=None, tp_rank=0):
    """Forward of the unsharded block given as R shards.

    x [B, S, H]; w the unsharded weights (keys as in the inputs module:
    wq [nq*d, H], wk, wv [nkv*d, H], wo [H, nq*d], w1 [F, H] or wg, wu [F, H],
    w2 [H, F], optional biases and LN gain/shift). q_heads, kv_heads are the
    unsharded head counts; each of the R shards takes q_heads/R and
    kv_heads/R whole heads and ffn/R MLP columns. norm = "pre" (LN before
    each sublayer) or "post" (LN after each residual sum). Returns
    (out, cache). dropout: None or dict(p_attn, p_hidden, seed, offset); shard
    r of the R is tensor-parallel rank tp_rank + r (its attention seed)."""
    if norm not in ("pre", "post"):
        raise ValueError(norm)
    post = norm == "post"
    dr = dict(p_attn=0.0, p_hidden=0.0, seed=0, offset=0) if dropout is None else dict(dropout)
    x = np.asarray(x, F64)
    w = {k: np.asarray(v, F64) for k, v in w.items()}
    B, S, H = x.shape
    T = B * S
    d = head_dim
    nq, nkv = q_heads // R, kv_heads // R
    x2 = x.reshape(T, H)
    cache = {"R": R, "B": B, "S": S, "H": H, "nq": nq, "nkv": nkv, "d": d,
             "act": act, "causal": causal, "x": x2, "w": w, "shards": [], "post": post}

    if post:
        a = x2          # post-LN: attention reads the block input itself
    else:
        # (2) input LayerNorm, replicated on every rank
        a, xhat1, rstd1 = layer_norm_fwd(x2, w.get("ln1_g"), w.get("ln1_b"), eps)
        cache.update(xhat1=xhat1, rstd1=rstd1)
    cache["a"] = a

    # attention: each shard owns whole heads; its projection is a partial sum
    p_attn = []
    for r in range(R):
        ws = shard(w, R, r, d)
        q = _lin(a, ws["wq"], ws.get("bq")).reshape(B, S, nq, d).transpose(0, 2, 1, 3)
        k = _lin(a, ws["wk"], ws.get("bk")).reshape(B, S, nkv, d).transpose(0, 2, 1, 3)
        v = _lin(a, ws["wv"], ws.get("bv")).reshape(B, S, nkv, d).transpose(0, 2, 1, 3)
        mult = None
        if dr["p_attn"] > 0.0:
            mult = odrop.AttnMult(B, nq, S, odrop.attn_seed(dr["seed"], tp_rank + r),
                                  dr["offset"], dr["p_attn"])
        o = attention_fwd(q, k, v, causal, mult)
        o_tok = o.transpose(0, 2, 1, 3).reshape(T, nq * d)
        p_attn.append(o_tok @ ws["wo"].T)
        cache["shards"].append({"w": ws, "q": q, "k": k, "v": v, "o": o_tok, "mult": mult})
    cache["p_attn"] = p_attn

    # reduction point g1 (sum of partials), bias once, (4) residual
    attn = sum(p_attn)
    if "bo" in w:
        attn = attn + w["bo"]
    # hidden dropout outside the TP region: the same mask on every rank
    mult_h1 = odrop.multiplier((T, H), odrop.SITE_HIDDEN_ATTN, dr["seed"], dr["offset"],
                               dr["p_hidden"])
    mult_h2 = odrop.multiplier((T, H), odrop.SITE_HIDDEN_MLP, dr["seed"], dr["offset"],
                               dr["p_hidden"])
    cache.update(mult_h1=mult_h1, mult_h2=mult_h2)
    attn = attn * mult_h1
    if post:
        # residual first, then the first LayerNorm; the MLP reads its output
        h, xhat1, rstd1 = layer_norm_fwd(x2 + attn, w.get("ln1_g"), w.get("ln1_b"), eps)
        c = h
        cache.update(h=h, c=c, xhat1=xhat1, rstd1=rstd1)
    else:
        h = x2 + attn
        # (5) second LayerNorm
        c, xhat2, rstd2 = layer_norm_fwd(h, w.get("ln2_g"), w.get("ln2_b"), eps)
        cache.update(h=h, c=c, xhat2=xhat2, rstd2=rstd2)

    # MLP: column-parallel fc1 + activation, row-parallel fc2 partials
    p_mlp = []
    for r in range(R):
        sh = cache["shards"][r]
        ws = sh["w"]
        if act == "gelu":
            u = _lin(c, ws["w1"], ws.get("b1"))
            m = gelu(u)
            sh.update(u=u, m=m)
        else:
            ug = _lin(c, ws["wg"], ws.get("bg"))
            uu = _lin(c, ws["wu"], ws.get("bu"))
            m = swiglu(ug, uu)
            sh.update(ug=ug, uu=uu, m=m)
        p_mlp.append(m @ ws["w2"].T)
    cache["p_mlp"] = p_mlp

    # (6) reduction point g2, bias once, (7) residual
    y = sum(p_mlp)
    if "b2" in w:
        y = y + w["b2"]
    y = y * mult_h2
    if post:
        out, xhat2, rstd2 = layer_norm_fwd(h + y, w.get("ln2_g"), w.get("ln2_b"), eps)
        cache.update(xhat2=xhat2, rstd2=rstd2)
    else:
        out = h + y
    return out.reshape(B, S, H), cache


def block_backward(G, cache):
    """Backward of ``block_forward`` for the cotangent G = dL/d out [B, S, H].

    Returns (dx [B, S, H], grads) with grads holding the unsharded gradient
    of every weight present (shard slices concatenated back), plus the
    per-shard partials at the two backward reduction points under
    grads["_dc_partials"] and grads["_da_partials"], and the per-token key
    gradients (whose column sums give the key-bias gradient) under
    grads["_dk_tokens"]."""
    R, B, S, H = cache["R"], cache["B"], cache["S"], cache["H"]
    nq, nkv, d = cache["nq"], cache["nkv"], cache["d"]
    T = B * S
    w = cache["w"]
    G2 = np.asarray(G, F64).reshape(T, H)
    post = cache["post"]
    sg = {}
    if post:
        # post-LN: the output LayerNorm first; its input gradient feeds both
        # the MLP branch and the residual into h
        up, dg2, db2n = layer_norm_bwd(G2, cache["xhat2"], cache["rstd2"], w.get("ln2_g"))
    else:
        up = G2
    upm = up * cache["mult_h2"]     # through the MLP output's dropout

    # fc2 (row-parallel): g2's backward passes its upstream gradient unchanged
    # to every shard
    dc_parts = []
    for r in range(R):
        sh = cache["shards"][r]
        ws = sh["w"]
        g = {}
        dm = upm @ ws["w2"]
        g["w2"] = upm.T @ sh["m"]
        if cache["act"] == "gelu":
            du = dm * gelu_grad(sh["u"])
            g["w1"] = du.T @ cache["c"]
            if "b1" in ws:
                g["b1"] = du.sum(0)
            dc_parts.append(du @ ws["w1"])
        else:
            dug, duu = swiglu_grad(sh["ug"], sh["uu"], dm)
            g["wg"] = dug.T @ cache["c"]
            g["wu"] = duu.T @ cache["c"]
            if "bg" in ws:
                g["bg"] = dug.sum(0)
                g["bu"] = duu.sum(0)
            dc_parts.append(dug @ ws["wg"] + duu @ ws["wu"])
        sg[r] = g
    if "b2" in w:
        db2 = upm.sum(0)

    # column-parallel fc1 input: its gradient is summed over shards (f's backward)
    dc = sum(dc_parts)
    if post:
        dh = up + dc                        # at h = LN1(r1): residual + MLP input
        up_attn, dg1, db1n = layer_norm_bwd(dh, cache["xhat1"], cache["rstd1"], w.get("ln1_g"))
    else:
        dh_ln, dg2, db2n = layer_norm_bwd(dc, cache["xhat2"], cache["rstd2"], w.get("ln2_g"))
        dh = G2 + dh_ln
        up_attn = dh
    upa = up_attn * cache["mult_h1"]  # through the attention output's dropout

    # attention: projection (row-parallel), per-head attention, QKV (column-parallel)
    da_parts = []
    dk_tok = []
    for r in range(R):
        sh = cache["shards"][r]
        ws = sh["w"]
        g = sg[r]
        do_tok = upa @ ws["wo"]
        g["wo"] = upa.T @ sh["o"]
        do = do_tok.reshape(B, S, nq, d).transpose(0, 2, 1, 3)
        dq, dk, dv = attention_bwd(sh["q"], sh["k"], sh["v"], do, cache["causal"], sh["mult"])
        dq2 = dq.transpose(0, 2, 1, 3).reshape(T, nq * d)
        dk2 = dk.transpose(0, 2, 1, 3).reshape(T, nkv * d)
        dv2 = dv.transpose(0, 2, 1, 3).reshape(T, nkv * d)
        a = cache["a"]
        g["wq"], g["wk"], g["wv"] = dq2.T @ a, dk2.T @ a, dv2.T @ a
        if "bq" in ws:
            g["bq"], g["bk"], g["bv"] = dq2.sum(0), dk2.sum(0), dv2.sum(0)
        da_parts.append(dq2 @ ws["wq"] + dk2 @ ws["wk"] + dv2 @ ws["wv"])
        dk_tok.append(dk2)
    if "bo" in w:
        dbo = upa.sum(0)

    da = sum(da_parts)
    if post:
        dx = up_attn + da                   # attention read x itself
    else:
        dx_ln, dg1, db1n = layer_norm_bwd(da, cache["xhat1"], cache["rstd1"], w.get("ln1_g"))
        dx = dh + dx_ln

    grads = {}
    for k in sg[0]:
        axis = 1 if k in _ROW else 0
        grads[k] = np.concatenate([sg[r][k] for r in range(R)], axis=axis)
    if "b2" in w:
        grads["b2"] = db2
    if "bo" in w:
        grads["bo"] = dbo
    if "ln1_g" in w:
        grads["ln1_g"], grads["ln2_g"] = dg1, dg2
    if "ln1_b" in w:
        grads["ln1_b"], grads["ln2_b"] = db1n, db2n
    grads["_dc_partials"] = dc_parts
    grads["_da_partials"] = da_parts
    grads["_dh"] = dh
    grads["_dk_tokens"] = np.concatenate(dk_tok, axis=1)   # [T, nkv*d] per-token key gradients
    return dx.reshape(B, S, H), grads


def block_loss_mean(out):
    """The listing's loss ([Lab06] sec. 2 step (8)): the mean over every
    element of out. Returns (loss, dL/d out); the gradient of a mean is
    1 / numel in every position, whatever out holds."""
    out = np.asarray(out, np.float64)
    return float(out.sum() / out.size), np.full(out.shape, 1.0 / out.size)
