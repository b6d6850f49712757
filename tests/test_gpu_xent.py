"""GPU parity of the vocab-parallel cross-entropy against the fp64 oracle.
All vocab shards are run one after another on one GPU; their statistics are
combined by mtb_vocab_xent_combine (the three reductions of [TP-block] sec. 4).
"""
import numpy as np
import pytest
import torch

from gpu_util import TOL, host, rel_err, say
from oracle import xent as ox
from transformer_layer_ln_amd import inputs, mtb

pytestmark = pytest.mark.gpu


def _run_shards(shards, target, vocab, dtype, dloss):
    """shards: list of host [N, V_r] arrays -> (loss, stats, list of dz)."""
    dev = torch.device("cuda")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    code = mtb.BF16 if dtype == "bf16" else mtb.F32
    N = shards[0].shape[0]
    R = len(shards)
    tg = torch.as_tensor(target).to(dev)
    parts = torch.full((R, 3, N), float("nan"), device=dev)
    zs = []
    v0 = 0
    for r, z in enumerate(shards):
        zd = torch.as_tensor(z).to(dev, tdt).contiguous()
        zs.append((zd, v0))
        mtb.vocab_xent(N, z.shape[1], v0, code, mtb.XENT_PARTIAL, zd, tg, parts[r])
        v0 += z.shape[1]
    assert v0 == vocab
    stats = torch.empty(3, N, device=dev)
    loss = torch.empty(N, device=dev)
    mtb.vocab_xent_combine(N, R, parts, stats, loss)
    dl = torch.as_tensor(dloss).to(dev)
    dzs = []
    for zd, a in zs:
        dz = torch.full_like(zd, float("nan"))
        mtb.vocab_xent(N, zd.shape[1], a, code, mtb.XENT_FINISH, zd, tg, stats, None, dl, dz)
        dzs.append(dz)
    torch.cuda.synchronize()
    return host(loss), host(stats), [host(d) for d in dzs]


def _oracle(shards, target, dloss):
    v0s = np.cumsum([0] + [z.shape[1] for z in shards[:-1]])
    loss, gmax, sexp = ox.vocab_parallel_xent(shards, target, v0s)
    dz = [ox.vocab_parallel_xent_bwd(z, target, a, gmax, sexp, dloss) for z, a in zip(shards, v0s)]
    return loss, dz


@pytest.mark.parametrize("dtype,N,V,R", [
    ("bf16", 37, 8 * 264, 8),     # shard width multiple of 8: vector path
    ("bf16", 50, 3 * 1001, 3),    # odd shard width: scalar path
    ("f32", 33, 4 * 520, 4),
    ("f32", 20, 2 * 77, 2),
    ("bf16", 9, 1 * 4000, 1),     # one shard = the whole vocab
])
def test_sharded_xent_matches_oracle(dtype, N, V, R):
    say(f"[gpu] xent {dtype} N={N} V={V} R={R}")
    rng = np.random.default_rng(N * V)
    z = rng.standard_normal((N, V)).astype(np.float32) * 3
    if dtype == "bf16":
        z = inputs.round_bf16(z)
    y = rng.integers(0, V, N)
    vr = V // R
    y[:R] = np.arange(R) * vr                    # first id of each shard
    y[R:2 * R] = np.arange(R) * vr + vr - 1      # last id of each shard
    dl = rng.standard_normal(N).astype(np.float32)
    shards = [z[:, r * vr:(r + 1) * vr] for r in range(R)]
    loss, _, dz = _run_shards(shards, y, V, dtype, dl)
    ref_loss, ref_dz = _oracle(shards, y, dl)
    tol = TOL[dtype]
    assert rel_err(loss, ref_loss) <= tol
    assert rel_err(np.concatenate(dz, 1), np.concatenate(ref_dz, 1)) <= tol


def test_xent_all_phase_single_shard_and_in_place_gradient():
    N, V = 64, 1024
    say(f"[gpu] xent ALL N={N} V={V}")
    rng = np.random.default_rng(3)
    z = inputs.round_bf16(rng.standard_normal((N, V)).astype(np.float32))
    y = rng.integers(0, V, N)
    dl = np.full(N, 1.0 / N, np.float32)
    dev = torch.device("cuda")
    zd = torch.as_tensor(z).to(dev, torch.bfloat16).contiguous()
    stats = torch.empty(4, N, device=dev)
    loss = torch.empty(N, device=dev)
    mtb.vocab_xent(N, V, 0, mtb.BF16, mtb.XENT_ALL, zd, torch.as_tensor(y).to(dev), stats, loss,
                   torch.as_tensor(dl).to(dev), zd)          # gradient written over the logits
    torch.cuda.synchronize()
    ref_loss, ref_dz = _oracle([z], y, dl)
    assert rel_err(host(loss), ref_loss) <= 2e-2
    assert rel_err(host(zd), ref_dz[0]) <= 2e-2


def test_xent_all_phase_calls_hook_max_sum_sum():
    N, V = 16, 512
    calls = []

    def cb(buf, count, dtype, op, stream, user):
        calls.append((count, dtype, op))
        return 0

    fn = mtb.ALLREDUCE_FN(cb)
    comm = mtb.Comm(fn, None)
    dev = torch.device("cuda")
    rng = np.random.default_rng(4)
    z = rng.standard_normal((N, V)).astype(np.float32)
    y = rng.integers(0, V, N)
    say("[gpu] xent hook order")
    zd = torch.as_tensor(z).to(dev)
    stats = torch.empty(4, N, device=dev)
    loss = torch.empty(N, device=dev)
    mtb.vocab_xent(N, V, 0, mtb.F32, mtb.XENT_ALL, zd, torch.as_tensor(y).to(dev), stats, loss,
                   comm=comm)
    torch.cuda.synchronize()
    assert calls == [(N, mtb.F32, mtb.OP_MAX), (N, mtb.F32, mtb.OP_SUM), (N, mtb.F32, mtb.OP_SUM)]
    ref_loss, _ = _oracle([z], y, np.zeros(N))
    assert rel_err(host(loss), ref_loss) <= 1e-4


def test_c5_vocab_shards_full_size():
    """8 shards of [8192, 16032] bf16 logits (vocab 128256): loss on every
    token, gradient on a sample of rows in every shard."""
    cfg = inputs.C5_XENT
    say(f"[gpu] xent {cfg.name}")
    y = inputs.xent_targets(cfg)
    dl = inputs.xent_dloss(cfg)
    shards = [inputs.xent_logits(cfg, r) for r in range(cfg.tp)]
    loss, stats, dz = _run_shards(shards, y, cfg.vocab, cfg.dtype, dl)
    rows = np.random.default_rng(0).choice(cfg.n_tokens, 256, replace=False)
    v0s = [r * cfg.v_local for r in range(cfg.tp)]
    # oracle: loss over all tokens, streamed shard by shard as the page's reductions go
    gmax = np.max(np.stack([ox.local_max(z) for z in shards]), axis=0)
    sums = [ox.local_sums(z, y, a, gmax) for z, a in zip(shards, v0s)]
    sexp = np.sum([s for s, _ in sums], axis=0)
    pred = np.sum([p for _, p in sums], axis=0)
    ref_loss = np.log(sexp) - pred
    assert rel_err(loss, ref_loss) <= TOL["bf16"]
    for r in range(cfg.tp):
        ref = ox.vocab_parallel_xent_bwd(shards[r][rows], y[rows], v0s[r], gmax[rows], sexp[rows], dl[rows])
        assert rel_err(dz[r][rows], ref) <= TOL["bf16"], r
