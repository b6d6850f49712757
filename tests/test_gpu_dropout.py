"""GPU parity of the block with tensor-parallel dropout ([TP-block] sec. 5)
against the fp64 oracle: attention-probability masks from this rank's stream
(seed + 2718 + tp_rank), hidden-state masks after the attention and after the
MLP from the shared seed. The GPU and the oracle each implement the
counter-based generator; a single differing mask bit would show as an O(1)
error, so the fp32 cases at 1e-4 check the masks bit for bit in effect.

The probabilities are dyadic (0.25, 0.125, 0.375) so that the float in
mtb_cfg and the oracle's Python float give the same integer threshold.
"""
import numpy as np
import pytest

from gpu_util import check_rank_vs_oracle, rel_err, run_rank, say
from transformer_layer_ln_amd import inputs, mtb

pytestmark = pytest.mark.gpu

DROP = dict(p_attn=0.25, p_hidden=0.125, drop_seed=0x5EED5EED1234, drop_offset=3)


def _case(cfg):
    a = inputs.activations(cfg)
    return inputs.shard_weights(cfg, 0), a["x"], a["g"]


@pytest.mark.parametrize("variant,rank", [
    (dict(), 0),
    (dict(causal=True, affine=True, bias=True), 3),
    (dict(act="swiglu", ffn=256, kv_heads=2, norm="post", bias=True), 1),
    (dict(p_hidden=0.0), 5),
    (dict(p_attn=0.0, p_hidden=0.375, norm="post"), 0),
])
def test_fp32_dropout(variant, rank):
    cfg = inputs.C1.with_(name="fp32-dropout", **dict(DROP, **variant))
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G, tp_rank=rank)


BF16 = [
    dict(batch=2, seq=192, hidden=192, q_heads=2, kv_heads=2, head_dim=64, ffn=320),
    dict(batch=2, seq=256, hidden=256, q_heads=4, kv_heads=2, head_dim=128, ffn=384, causal=True,
         act="swiglu", bias=True, affine=True),
    dict(batch=1, seq=320, hidden=256, q_heads=2, kv_heads=1, head_dim=64, ffn=256, causal=True,
         norm="post"),
]


@pytest.mark.parametrize("i", range(len(BF16)))
def test_bf16_dropout(i):
    cfg = inputs.BlockConfig(f"bf16-dropout-{i}", dtype="bf16", tp=1, seed=2800 + i,
                             **dict(DROP, **BF16[i]))
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G, tp_rank=2 + i)


def test_dropout_is_reproducible_and_rank_dependent():
    cfg = inputs.BlockConfig("drop-det", batch=2, seq=128, hidden=256, q_heads=2, kv_heads=2,
                             head_dim=64, ffn=256, causal=True, seed=2900, **DROP)
    w, x, G = _case(cfg)
    say("[gpu] dropout: same seed -> same bits; another rank -> another attention mask")
    r1 = run_rank(cfg, w, x, G, tp_rank=1)
    r2 = run_rank(cfg, w, x, G, tp_rank=1)
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    for k in r1[2]:
        assert np.array_equal(r1[2][k], r2[2][k]), k
    r3 = run_rank(cfg, w, x, G, tp_rank=2)
    assert rel_err(r3[0], r1[0]) > 1e-2
    # attention dropout off: the rank no longer matters
    c0 = cfg.with_(p_attn=0.0)
    a = run_rank(c0, w, x, G, tp_rank=1)
    b = run_rank(c0, w, x, G, tp_rank=6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # another offset: other masks
    r4 = run_rank(cfg.with_(drop_offset=4), w, x, G, tp_rank=1)
    assert rel_err(r4[0], r1[0]) > 1e-2


def test_dropout_hook_path_matches_oracle():
    """MTB_PHASE_ALL with a reduction hook runs the hidden dropout in the
    LayerNorm / add kernels after the reduction instead of the GEMM
    epilogue: the same masks, checked against the oracle."""
    cfg = inputs.BlockConfig("drop-hook", batch=2, seq=128, hidden=256, q_heads=2, kv_heads=2,
                             head_dim=64, ffn=256, seed=2910, bias=True, **DROP)
    w, x, G = _case(cfg)
    calls = []
    fn = mtb.ALLREDUCE_FN(lambda buf, count, dtype, op, stream, user: calls.append(op) or 0)
    comm = mtb.Comm(fn, None)
    for norm in ("pre", "post"):
        c = cfg.with_(norm=norm)
        check_rank_vs_oracle(c, w, x, G, comm=comm, tp_rank=1, label=f"dropout, hook, {norm}-LN")
    assert len(calls) == 8


@pytest.mark.timeout(400)
def test_seq2048_share_with_dropout_full_size():
    """The workload `bench.py --workload seq2048-dropout` times: the seq-2048
    causal TP=8 rank share with dropout 0.1 on all three sites, whole
    tensors. p is taken as its float32 value on both sides (the device
    threshold comes from the float in mtb_cfg). The oracle's masks alone are
    ~10^8 generator words: tens of seconds on the CPU."""
    p = float(np.float32(0.1))
    cfg = inputs.C4.with_(name="C4-dropout", p_attn=p, p_hidden=p, drop_seed=1234, drop_offset=0)
    w, x, G = _case(cfg)
    check_rank_vs_oracle(cfg, w, x, G, tp_rank=3)
