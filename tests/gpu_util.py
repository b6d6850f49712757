"""Helpers shared by the GPU parity tests: run the block through the C ABI on
seeded inputs and compare element by element with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import block as ob
from transformer_layer_ln_amd import inputs, mtb

TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    """Name the case on stdout before any GPU work (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def rel_err(gpu, ref):
    """max |gpu - ref| / max |ref| over a whole tensor."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite values"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def elem_err(gpu, ref, floor=1e-3):
    """Largest elementwise relative error, each element's |ref| floored at
    floor * max|ref| (a plain elementwise ratio is undefined where ref is 0).
    Logged beside rel_err, which is what the tolerance applies to: it shows
    errors concentrated in the small entries of a tensor."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.max(np.abs(ref))
    den = np.maximum(np.abs(ref), floor * (m if m > 0 else 1.0))
    return float(np.max(np.abs(gpu - ref) / den))


def zero_sum_err(gpu, terms):
    """Error of a gradient that is exactly zero in exact arithmetic (the key
    bias: softmax ignores a shift shared by a whole row of scores), measured
    against the sum of the magnitudes of the per-token terms that cancel."""
    scale = np.max(np.sum(np.abs(np.asarray(terms, np.float64)), axis=0))
    # every term zero (a single key per query: softmax has no score gradient):
    # what the GPU leaves is rounding residue, judged in absolute terms
    return float(np.max(np.abs(np.asarray(gpu, np.float64))) / (scale if scale > 0 else 1.0))


def host(t):
    return t.detach().float().cpu().numpy()


def oracle_kw(cfg):
    kw = dict(q_heads=cfg.q_heads, kv_heads=cfg.kv_heads, head_dim=cfg.head_dim, act=cfg.act,
              causal=cfg.causal, eps=cfg.ln_eps, norm=cfg.norm)
    if cfg.p_attn or cfg.p_hidden:
        kw["dropout"] = dict(p_attn=cfg.p_attn, p_hidden=cfg.p_hidden, seed=cfg.drop_seed,
                             offset=cfg.drop_offset)
    return kw


def split_grads(g: dict, cfg) -> dict:
    """ABI gradient tensors -> the oracle's split names (host fp32/64)."""
    d, nq, nkv = cfg.head_dim, cfg.q_heads, cfg.kv_heads
    out = {}
    if "w_qkv" in g:
        a = host(g["w_qkv"])
        out["wq"], out["wk"], out["wv"] = a[:nq * d], a[nq * d:(nq + nkv) * d], a[(nq + nkv) * d:]
    if "b_qkv" in g:
        a = host(g["b_qkv"])
        out["bq"], out["bk"], out["bv"] = a[:nq * d], a[nq * d:(nq + nkv) * d], a[(nq + nkv) * d:]
    if "w_o" in g:
        out["wo"] = host(g["w_o"])
    if "b_o" in g:
        out["bo"] = host(g["b_o"])
    if "w_fc2" in g:
        out["w2"] = host(g["w_fc2"])
    if "b_fc2" in g:
        out["b2"] = host(g["b_fc2"])
    if "w_fc1" in g:
        if cfg.act == "gelu":
            out["w1"] = host(g["w_fc1"])
        else:
            a, b = mtb.split_gate_up(g["w_fc1"])
            out["wg"], out["wu"] = host(a), host(b)
    if "b_fc1" in g:
        if cfg.act == "gelu":
            out["b1"] = host(g["b_fc1"])
        else:
            a, b = mtb.split_gate_up(g["b_fc1"])
            out["bg"], out["bu"] = host(a), host(b)
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        if k in g:
            out[k] = host(g[k])
    return out


def run_rank(cfg, w_split, x, G, comm=None, tp_rank=0):
    """Forward + backward of one rank's share with MTB_PHASE_ALL.
    Returns (out, dx, grads-in-oracle-names) on the host."""
    dev = torch.device("cuda")
    dt = tdtype(cfg)
    c = mtb.cfg_from(cfg, tp_rank)
    w = mtb.device_weights(w_split, cfg.act, dt, dev)
    blk = mtb.BlockShard(c, w, dev)
    xd = torch.as_tensor(x).to(dev, dt).contiguous()
    Gd = torch.as_tensor(G).to(dev, dt).contiguous()
    out = torch.full_like(xd, float("nan"))
    dx = torch.full_like(xd, float("nan"))
    grads = {k: torch.full_like(v, float("nan")) for k, v in w.items()}
    blk.fwd(xd, out, comm=comm)
    blk.bwd(xd, Gd, dx, grads, comm=comm)
    torch.cuda.synchronize()
    return host(out), host(dx), split_grads(grads, cfg)


def check_rank_vs_oracle(cfg, w_split, x, G, tol=None, comm=None, label="", tp_rank=0):
    tol = TOL[cfg.dtype] if tol is None else tol
    say(f"[gpu] {label or cfg.name}: B={cfg.batch} S={cfg.seq} H={cfg.hidden} nq={cfg.q_heads} "
        f"nkv={cfg.kv_heads} d={cfg.head_dim} F={cfg.ffn} act={cfg.act} causal={cfg.causal} "
        f"dtype={cfg.dtype} norm={cfg.norm} dropout={cfg.p_attn}/{cfg.p_hidden} rank={tp_rank}")
    out, dx, grads = run_rank(cfg, w_split, x, G, comm=comm, tp_rank=tp_rank)
    ref_out, cache = ob.block_forward(x, w_split, R=1, tp_rank=tp_rank, **oracle_kw(cfg))
    ref_dx, ref_g = ob.block_backward(G, cache)
    errs = {"out": rel_err(out, ref_out), "dx": rel_err(dx, ref_dx)}
    elem = {"out": elem_err(out, ref_out), "dx": elem_err(dx, ref_dx)}
    for k in w_split:
        errs[k] = rel_err(grads[k], ref_g[k]) if k != "bk" else zero_sum_err(grads[k], ref_g["_dk_tokens"])
        if k != "bk":
            elem[k] = elem_err(grads[k], ref_g[k])
    say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    say("   elementwise (floor 1e-3 max|ref|, logged only):", {k: f"{v:.2e}" for k, v in elem.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"above tolerance {tol}: {bad}"
    return errs
