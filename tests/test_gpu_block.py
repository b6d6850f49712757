"""GPU parity of the block forward + backward (through the C ABI) against the
fp64 oracle on identical seeded inputs.

Tolerance (per output tensor, max |gpu - ref| / max |ref|): 2e-2 for bf16,
1e-4 for fp32. The cotangent is a seeded N(0,1) tensor G (a row-constant
cotangent such as mean(out)'s would leave part of the LayerNorm backward
unexercised), plus one run with the listing's own loss = mean(out).
"""
import numpy as np
import pytest

from gpu_util import TOL, check_rank_vs_oracle, host, rel_err, run_rank, say, tdtype
from oracle import block as ob
from transformer_layer_ln_amd import inputs, mtb

pytestmark = pytest.mark.gpu


def _case(cfg):
    a = inputs.activations(cfg)
    return inputs.shard_weights(cfg, 0), a["x"], a["g"]


def test_c1_fp32_full_block():
    cfg = inputs.C1
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


def test_c1_fp32_mean_loss():
    """The listing's loss: out.mean(); its cotangent (1/numel) comes from the
    oracle's loss function."""
    cfg = inputs.C1
    w, x, _ = _case(cfg)
    _, G = ob.block_loss_mean(x)   # the cotangent does not depend on the values
    G = G.astype(x.dtype)
    check_rank_vs_oracle(cfg, w, x, G, label="C1 mean(out)")


@pytest.mark.parametrize("variant", [
    dict(causal=True),
    dict(act="swiglu", ffn=256, kv_heads=2),
    dict(act="swiglu", ffn=256, kv_heads=1, causal=True, affine=True, bias=True),
    dict(affine=True, bias=True, seq=40, head_dim=64, q_heads=2, kv_heads=2),
])
def test_fp32_variants(variant):
    cfg = inputs.C1.with_(name="fp32-variant", **variant)
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


# bf16: shapes with ragged tails against the 128-wide GEMM tiles and the
# 128-query attention tiles (seq 192, hidden 192/320, ffn 320, 3 heads)
BF16_SMALL = [
    dict(batch=3, seq=192, hidden=192, q_heads=2, kv_heads=2, head_dim=64, ffn=320),
    dict(batch=2, seq=192, hidden=320, q_heads=3, kv_heads=1, head_dim=64, ffn=192, causal=True,
         act="swiglu", affine=True, bias=True),
    dict(batch=2, seq=256, hidden=256, q_heads=2, kv_heads=2, head_dim=128, ffn=384, causal=True),
    dict(batch=1, seq=320, hidden=256, q_heads=4, kv_heads=2, head_dim=128, ffn=256, act="swiglu",
         bias=True),
    dict(batch=2, seq=64, hidden=128, q_heads=1, kv_heads=1, head_dim=64, ffn=64, causal=True),
]


@pytest.mark.parametrize("i", range(len(BF16_SMALL)))
def test_bf16_small_shapes(i):
    cfg = inputs.BlockConfig(f"bf16-small-{i}", dtype="bf16", tp=1, seed=2000 + i, **BF16_SMALL[i])
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


# Shapes that reach the hand-scheduled 256 x 256 GEMM (contractions that are
# multiples of 32 and at least 1024 deep) with ragged edges: 4032 tokens
# (fc1 forward, fc2 dgrad: token rows past the last full tile), and ragged
# weight dimensions 2112 x 1344 for the weight gradients, whose contraction
# (4096 tokens) is split four ways; hidden 1984 (a 192-wide last tile), where
# the QKV and projection weight gradients run as one grouped launch (1536 x
# 1984 and 1984 x 512, each split four ways: 192 + 64 blocks); 8064 tokens at
# hidden 1984 with biases, where fc2 and the 512-deep projection forward add
# their residual rows on the scheduled kernel past both ragged edges (a
# 128-row last tile row, a 192-wide last tile column) and the grouped weight
# gradients split 8064 tokens four ways (63 k-tiles each, entering the loop
# body at its second slot); SwiGLU at 4032 tokens, where the SwiGLU′ epilogue
# of the fc2 data gradient takes its prefetched gate/up rows past the last
# full tile row. 8064 tokens with a 3584-wide GELU fc1 (448 tiles of 256 x
# 256) split its columns into 2048 on 256 x 256 tiles and 1536 on 256 x 192
# tiles, past a ragged last tile row.
SCHED_RAGGED = [
    dict(batch=3, seq=1344, hidden=1280, q_heads=10, kv_heads=2, head_dim=128, ffn=3072, causal=True),
    dict(batch=2, seq=2048, hidden=1344, q_heads=21, kv_heads=3, head_dim=64, ffn=2112, bias=True,
         affine=True),
    dict(batch=2, seq=2048, hidden=1984, q_heads=4, kv_heads=4, head_dim=128, ffn=576, causal=True),
    dict(batch=3, seq=2688, hidden=1984, q_heads=4, kv_heads=4, head_dim=128, ffn=576, causal=True,
         bias=True),
    dict(batch=3, seq=1344, hidden=1280, q_heads=10, kv_heads=2, head_dim=128, ffn=3072, act="swiglu",
         causal=True),
    dict(batch=3, seq=2688, hidden=256, q_heads=2, kv_heads=2, head_dim=128, ffn=3584, causal=True, bias=True),
]


@pytest.mark.parametrize("i", range(len(SCHED_RAGGED)))
def test_bf16_scheduled_gemm_ragged_shapes(i):
    cfg = inputs.BlockConfig(f"bf16-sched-ragged-{i}", dtype="bf16", tp=1, seed=2100 + i, **SCHED_RAGGED[i])
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


def test_c2_rank_share():
    cfg = inputs.C2
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


def test_c4_rank_share_full_size():
    """The seq-2048 causal TP=8 rank share at its full size, whole tensors."""
    cfg = inputs.C4
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


def test_c5_swiglu_gqa_rank_share_full_size():
    cfg = inputs.C5
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


def test_gpu_results_are_deterministic():
    cfg = inputs.BlockConfig("det", batch=2, seq=256, hidden=256, q_heads=4, kv_heads=1, head_dim=64,
                             ffn=256, act="swiglu", causal=True, seed=2100)
    w, x, G = _case(cfg)
    say("[gpu] determinism", cfg)
    r1 = run_rank(cfg, w, x, G)
    r2 = run_rank(cfg, w, x, G)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    for k in r1[2]:
        assert np.array_equal(r1[2][k], r2[2][k]), k


def _graph_case(cfg):
    """Eager fwd+bwd, then the same step captured in a HIP graph and replayed
    three times with eager work and synchronisations in between; every replay
    must reproduce the eager results bit for bit."""
    import torch

    w_split, x, G = _case(cfg)
    dev = torch.device("cuda")
    dt = torch.bfloat16
    blk = mtb.BlockShard(mtb.cfg_from(cfg), mtb.device_weights(w_split, cfg.act, dt, dev), dev)
    xd = torch.as_tensor(x).to(dev, dt)
    Gd = torch.as_tensor(G).to(dev, dt)
    out = torch.empty_like(xd)
    dx = torch.empty_like(xd)
    grads = blk.grad_buffers()
    blk.fwd(xd, out)
    blk.bwd(xd, Gd, dx, grads)
    torch.cuda.synchronize()
    ref = [out.clone(), dx.clone()] + [grads[k].clone() for k in sorted(grads)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        blk.fwd(xd, out)
        blk.bwd(xd, Gd, dx, grads)
    for rep in range(3):
        for t in [out, dx] + list(grads.values()):
            t.fill_(float("nan"))            # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [out, dx] + [grads[k] for k in sorted(grads)]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}, tensor {i}"
    say(f"   3 graph replays equal the eager step ({len(ref)} tensors)")


@pytest.mark.gpu
def test_graph_replay_matches_eager_step():
    cfg = inputs.BlockConfig("graph", batch=2, seq=256, hidden=512, q_heads=4, kv_heads=2,
                             head_dim=64, ffn=512, act="swiglu", causal=True, seed=2200)
    say("[gpu] graph replay", cfg)
    _graph_case(cfg)


@pytest.mark.gpu
def test_graph_replay_matches_eager_step_seq512_share():
    say("[gpu] graph replay, seq-512 TP=4 share")
    _graph_case(inputs.C2)


# post-LN ([Lab06] sec. 2 notes (2)(5)): residual first, then LayerNorm
@pytest.mark.parametrize("variant", [
    dict(),
    dict(act="swiglu", ffn=256, kv_heads=2, causal=True, affine=True, bias=True),
])
def test_fp32_post_ln(variant):
    cfg = inputs.C1.with_(name="fp32-post", norm="post", **variant)
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


@pytest.mark.parametrize("i", [0, 1, 3])
def test_bf16_post_ln_small_shapes(i):
    cfg = inputs.BlockConfig(f"bf16-post-{i}", dtype="bf16", tp=1, seed=2500 + i, norm="post",
                             **BF16_SMALL[i])
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


def test_c4_post_ln_rank_share_full_size():
    """The seq-2048 causal TP=8 rank share in post-LN order, whole tensors."""
    cfg = inputs.C4.with_(name="C4-post", norm="post")
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


@pytest.mark.gpu
def test_graph_replay_matches_eager_step_post_ln():
    cfg = inputs.BlockConfig("graph-post", batch=2, seq=256, hidden=512, q_heads=4, kv_heads=2,
                             head_dim=64, ffn=512, act="swiglu", causal=True, seed=2600, norm="post",
                             affine=True, bias=True)
    say("[gpu] graph replay, post-LN", cfg)
    _graph_case(cfg)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_largest_supported_hidden(dtype):
    """hidden = 8192, the largest the LayerNorm kernels hold in registers (16
    chunks of 8 per lane), with a short sequence so the oracle stays fast."""
    extra = dict(head_dim=64, q_heads=2, kv_heads=2) if dtype == "bf16" else dict(head_dim=32,
                                                                                  q_heads=2,
                                                                                  kv_heads=1)
    cfg = inputs.BlockConfig(f"hidden8192-{dtype}", batch=1, seq=64, hidden=8192, ffn=128,
                             dtype=dtype, causal=True, affine=True, bias=True, seed=2990, **extra)
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)


@pytest.mark.parametrize("seq", [1, 3])
def test_fp32_degenerate_sequences(seq):
    """One or three tokens per sequence (fp32 path: any seq): softmax over a
    single key, causal triangle of three."""
    cfg = inputs.C1.with_(name=f"fp32-seq{seq}", seq=seq, batch=3, causal=True, bias=True)
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G)
