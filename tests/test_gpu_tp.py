"""Tensor-parallel emulation on one GPU: all R rank shares of a layer run one
after another through the phase entry points, the test sums their partials
at the reduction points (the collectives of [TP-block] sec. 2), and the
result must equal the unsharded oracle block. Also covers the reduction hook
of MTB_PHASE_ALL."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import (TOL, check_rank_vs_oracle, host, oracle_kw, rel_err, run_rank, say, split_grads,
                      tdtype, zero_sum_err)
from oracle import block as ob
from transformer_layer_ln_amd import inputs, mtb

pytestmark = pytest.mark.gpu


def _sum(parts, dt):
    acc = torch.zeros_like(parts[0], dtype=torch.float32)
    for p in parts:
        acc += p.float()
    return acc.to(dt)


def emulate_tp(cfg):
    """Run the cfg.tp shards sequentially; return host out, dx, per-rank grads
    and the per-rank partials."""
    dev = torch.device("cuda")
    dt = tdtype(cfg)
    R = cfg.tp
    a = inputs.activations(cfg)
    x = torch.as_tensor(a["x"]).to(dev, dt).contiguous()
    G = torch.as_tensor(a["g"]).to(dev, dt).contiguous()
    shards = []
    for r in range(R):
        w = mtb.device_weights(inputs.shard_weights(cfg, r), cfg.act, dt, dev)
        shards.append(mtb.BlockShard(mtb.cfg_from(cfg, tp_rank=r), w, dev))
    buf = lambda: torch.full_like(x, float("nan"))
    # forward: SEG0 -> sum -> SEG1 -> sum -> SEG2
    p_attn = [buf() for _ in range(R)]
    for r, s in enumerate(shards):
        s.fwd(x, p_attn[r], phase=mtb.PHASE_SEG0)
    red1 = _sum(p_attn, dt)
    p_mlp = [buf() for _ in range(R)]
    for r, s in enumerate(shards):
        s.fwd(x, p_mlp[r], phase=mtb.PHASE_SEG1, reduced_in=red1)
    red2 = _sum(p_mlp, dt)
    outs = [buf() for _ in range(R)]
    for r, s in enumerate(shards):
        s.fwd(x, outs[r], phase=mtb.PHASE_SEG2, reduced_in=red2)
    # backward: SEG0 -> sum dc -> SEG1 -> sum da -> SEG2
    grads = [s.grad_buffers() for s in shards]
    dc = [buf() for _ in range(R)]
    for r, s in enumerate(shards):
        s.bwd(x, G, dc[r], grads[r], phase=mtb.PHASE_SEG0)
    red3 = _sum(dc, dt)
    da = [buf() for _ in range(R)]
    for r, s in enumerate(shards):
        s.bwd(x, G, da[r], grads[r], phase=mtb.PHASE_SEG1, reduced_in=red3)
    red4 = _sum(da, dt)
    dxs = [buf() for _ in range(R)]
    for r, s in enumerate(shards):
        s.bwd(x, G, dxs[r], grads[r], phase=mtb.PHASE_SEG2, reduced_in=red4)
    torch.cuda.synchronize()
    return dict(outs=[host(o) for o in outs], dxs=[host(d) for d in dxs],
                grads=[split_grads(g, cfg) for g in grads],
                p_attn=[host(p) for p in p_attn], p_mlp=[host(p) for p in p_mlp],
                dc=[host(p) for p in dc], da=[host(p) for p in da], x=a["x"], g=a["g"])


def _check_tp(cfg):
    say(f"[gpu] TP emulation {cfg.name}: R={cfg.tp} B={cfg.batch} S={cfg.seq} H={cfg.hidden}")
    res = emulate_tp(cfg)
    full = cfg.full()
    wf = inputs.full_weights(cfg)
    ref_out, cache = ob.block_forward(res["x"], wf, R=cfg.tp, **oracle_kw(full))
    ref_dx, ref_g = ob.block_backward(res["g"], cache)
    tol = TOL[cfg.dtype]
    errs = {}
    # every rank ends with the same replicated output and input gradient
    for r in range(cfg.tp):
        assert np.array_equal(res["outs"][r], res["outs"][0])
        assert np.array_equal(res["dxs"][r], res["dxs"][0])
    errs["out"] = rel_err(res["outs"][0], ref_out)
    errs["dx"] = rel_err(res["dxs"][0], ref_dx)
    # per-rank partials at the four reduction points
    B, S, H = cfg.batch, cfg.seq, cfg.hidden
    for r in range(cfg.tp):
        errs[f"p_attn{r}"] = rel_err(res["p_attn"][r].reshape(-1, H), cache["p_attn"][r])
        errs[f"p_mlp{r}"] = rel_err(res["p_mlp"][r].reshape(-1, H), cache["p_mlp"][r])
        errs[f"dc{r}"] = rel_err(res["dc"][r].reshape(-1, H), ref_g["_dc_partials"][r])
        errs[f"da{r}"] = rel_err(res["da"][r].reshape(-1, H), ref_g["_da_partials"][r])
    # weight gradients: rank r's slices of the unsharded gradient
    for k in res["grads"][0]:
        axis = 1 if k in ("wo", "w2") else 0
        if k in ("bo", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b"):
            got = res["grads"][0][k]
        else:
            got = np.concatenate([res["grads"][r][k] for r in range(cfg.tp)], axis=axis)
        errs["d" + k] = (rel_err(got, ref_g[k]) if k != "bk"
                         else zero_sum_err(got, ref_g["_dk_tokens"]))
    say("   errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"above tolerance {tol}: {bad}"


@pytest.mark.parametrize("seq", inputs.C3_SEQS)
def test_c3_four_shards_sum_to_unsharded_block(seq):
    _check_tp(inputs.C3(seq))


def test_tp_emulation_swiglu_gqa_with_biases_and_affine():
    cfg = inputs.BlockConfig("tp2-swiglu-gqa", batch=2, seq=128, hidden=256, q_heads=2, kv_heads=1,
                             head_dim=64, ffn=128, act="swiglu", causal=True, tp=2, seed=2200,
                             affine=True, bias=True)
    _check_tp(cfg)


def test_tp_emulation_fp32():
    cfg = inputs.C1.with_(name="tp2-fp32", q_heads=2, kv_heads=2, ffn=256, tp=2, bias=True)
    _check_tp(cfg)


def test_tp_emulation_post_ln_four_shards():
    _check_tp(inputs.C3(256).with_(name="C3-tp4-s256-post", norm="post"))


def test_tp_emulation_post_ln_swiglu_gqa_affine_fp32_and_bf16():
    cfg = inputs.BlockConfig("tp2-post", batch=2, seq=128, hidden=256, q_heads=2, kv_heads=1,
                             head_dim=64, ffn=128, act="swiglu", causal=True, tp=2, seed=2700,
                             affine=True, bias=True, norm="post")
    _check_tp(cfg)
    _check_tp(inputs.C1.with_(name="tp2-fp32-post", q_heads=2, kv_heads=2, ffn=256, tp=2,
                              bias=True, affine=True, norm="post"))


def test_tp_emulation_with_dropout():
    """[TP-block] sec. 5 across shards: each shard's attention masks come
    from its own rank's stream, the hidden masks (applied after the sums) are
    shared; the sum over shards must equal the oracle's R-shard block."""
    drop = dict(p_attn=0.25, p_hidden=0.125, drop_seed=77, drop_offset=1)
    _check_tp(inputs.C3(128).with_(name="C3-tp4-s128-dropout", **drop))
    _check_tp(inputs.C1.with_(name="tp2-fp32-dropout-post", q_heads=2, kv_heads=2, ffn=256, tp=2,
                              bias=True, norm="post", **drop))


class _Hook:
    """A reduction hook that records its calls and optionally fails."""

    def __init__(self, status=0):
        self.calls = []
        self.status = status
        self.fn = mtb.ALLREDUCE_FN(self._cb)
        self.comm = mtb.Comm(self.fn, None)

    def _cb(self, buf, count, dtype, op, stream, user):
        self.calls.append((count, dtype, op))
        return self.status


def test_reduction_hook_called_at_the_two_points_each_way():
    """MTB_PHASE_ALL with an (identity) hook runs the unfused LayerNorm / add
    kernels after each reduction point: checked against the oracle itself."""
    cfg = inputs.BlockConfig("hook", batch=2, seq=128, hidden=256, q_heads=2, kv_heads=2,
                             head_dim=64, ffn=256, seed=2300)
    a = inputs.activations(cfg)
    w = inputs.shard_weights(cfg, 0)
    hook = _Hook()
    check_rank_vs_oracle(cfg, w, a["x"], a["g"], comm=hook.comm, label="hook, identity")
    T, H = cfg.tokens, cfg.hidden
    assert hook.calls == [(T * H, mtb.BF16, mtb.OP_SUM)] * 4


def test_reduction_hook_post_ln_matches_oracle():
    cfg = inputs.BlockConfig("hook-post", batch=2, seq=128, hidden=256, q_heads=2, kv_heads=2,
                             head_dim=64, ffn=256, seed=2310, norm="post", affine=True, bias=True)
    a = inputs.activations(cfg)
    w = inputs.shard_weights(cfg, 0)
    hook = _Hook()
    check_rank_vs_oracle(cfg, w, a["x"], a["g"], comm=hook.comm, label="hook, identity, post-LN")
    T, H = cfg.tokens, cfg.hidden
    assert hook.calls == [(T * H, mtb.BF16, mtb.OP_SUM)] * 4


def test_reduction_hook_failure_is_reported():
    cfg = inputs.BlockConfig("hookfail", batch=1, seq=64, hidden=128, q_heads=2, kv_heads=2,
                             head_dim=64, ffn=128, seed=2400)
    a = inputs.activations(cfg)
    hook = _Hook(status=5)
    say("[gpu] reduction hook, failing")
    with pytest.raises(mtb.MtbError) as e:
        run_rank(cfg, inputs.shard_weights(cfg, 0), a["x"], a["g"], comm=hook.comm)
    assert e.value.status == mtb.MTB_ECOMM
    assert len(hook.calls) == 1
    torch.cuda.synchronize()
