"""Vocab-parallel input embedding on the GPU vs the fp64 oracle
([TP-block] sec. 3): per vocab shard, the masked lookup (bit-exact: it is a
copy) and the scatter-add backward (fp32 accumulation, one rounding)."""
import numpy as np
import pytest

from gpu_util import TOL, rel_err, say
from oracle import embed as oe
from transformer_layer_ln_amd import inputs, mtb

pytestmark = pytest.mark.gpu


def _run_shard(cfg, rank, check_bwd=True):
    import torch

    dev = torch.device("cuda")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    mdt = mtb.BF16 if cfg.dtype == "bf16" else mtb.F32
    n, h, vl = cfg.n_tokens, cfg.hidden, cfg.v_local
    v0 = rank * vl
    ids = inputs.embed_ids(cfg)
    table = inputs.embed_table(cfg, rank)
    ids_d = torch.as_tensor(ids).to(dev)
    tab_d = torch.as_tensor(table).to(dev, tdt)
    out = torch.full((n, h), float("nan"), dtype=tdt, device=dev)
    mtb.vocab_embed_fwd(n, vl, v0, h, mdt, ids_d, tab_d, out)
    torch.cuda.synchronize()
    ref = oe.embed_fwd(table, ids, v0)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref), f"forward shard {rank}"
    if not check_bwd:
        return
    dout = inputs.embed_dout(cfg)
    dout_d = torch.as_tensor(dout).to(dev, tdt)
    dtab = torch.full((vl, h), float("nan"), dtype=tdt, device=dev)
    ws = torch.empty(mtb.vocab_embed_bwd_workspace_bytes(n, vl), dtype=torch.uint8, device=dev)
    mtb.vocab_embed_bwd(n, vl, v0, h, mdt, ids_d, dout_d, dtab, ws)
    torch.cuda.synchronize()
    refb = oe.embed_bwd(dout, ids, v0, vl)
    gotb = dtab.float().cpu().numpy().astype(np.float64)
    hit = np.unique(ids[(ids >= v0) & (ids < v0 + vl)] - v0)
    untouched = np.setdiff1d(np.arange(vl), hit)
    assert not gotb[untouched].any(), "rows no token selects must be zero"
    err = rel_err(gotb, refb) if hit.size else 0.0
    say(f"   shard {rank}: {hit.size} rows hit, table-gradient error {err:.2e}")
    assert err <= TOL[cfg.dtype], (rank, err)
    # same inputs, same bits
    dtab2 = torch.empty_like(dtab)
    mtb.vocab_embed_bwd(n, vl, v0, h, mdt, ids_d, dout_d, dtab2, ws)
    torch.cuda.synchronize()
    assert torch.equal(dtab, dtab2)


@pytest.mark.parametrize("rank", [0, 7])
def test_embed_seq4096_vocab_shard_full_size(rank):
    cfg = inputs.C5_EMBED
    say(f"[gpu] embedding {cfg.name}, shard {rank}")
    _run_shard(cfg, rank)


def test_embed_forward_all_eight_shards_full_size():
    cfg = inputs.C5_EMBED
    say(f"[gpu] embedding forward, all shards of {cfg.name}")
    for r in range(cfg.tp):
        _run_shard(cfg, r, check_bwd=False)


@pytest.mark.parametrize("case", [
    dict(n_tokens=4099, vocab=1000, hidden=200, tp=4, repeat=37),   # heavy rows, ragged n and h
    dict(n_tokens=1, vocab=64, hidden=8, tp=2),
    dict(n_tokens=777, vocab=5000, hidden=264, tp=8, dtype="f32"),
    dict(n_tokens=16384, vocab=4096, hidden=128, tp=2, repeat=3),   # 3 ids, long scans
    dict(n_tokens=20000, vocab=600, hidden=2056, tp=2),             # > 2 column passes per row
])
def test_embed_variants(case):
    cfg = inputs.EmbedConfig("embed-var", seed=3100, **case)
    say(f"[gpu] embedding variant {case}")
    for r in sorted({0, cfg.tp - 1}):
        _run_shard(cfg, r)


def test_embed_ids_outside_every_shard():
    import torch

    dev = torch.device("cuda")
    ids = torch.tensor([-3, 0, 15, 16, 31, 1 << 40, -(1 << 40)], dtype=torch.int64, device=dev)
    table = torch.arange(16 * 8, dtype=torch.float32, device=dev).reshape(16, 8).to(torch.bfloat16)
    out = torch.full((7, 8), 7.0, dtype=torch.bfloat16, device=dev)
    mtb.vocab_embed_fwd(7, 16, 16, 8, mtb.BF16, ids, table, out)      # shard [16, 32)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    assert np.array_equal(o[3], table[0].float().cpu().numpy())
    assert np.array_equal(o[4], table[15].float().cpu().numpy())
    for t in (0, 1, 2, 5, 6):
        assert not o[t].any()


class _Hook:
    def __init__(self):
        self.calls = []
        self.fn = mtb.ALLREDUCE_FN(self._cb)
        self.comm = mtb.Comm(self.fn, None)

    def _cb(self, buf, count, dtype, op, stream, user):
        self.calls.append((count, dtype, op))
        return 0


def test_embed_forward_calls_the_reduction_hook_once():
    import torch

    dev = torch.device("cuda")
    ids = torch.tensor([1, 2, 3], dtype=torch.int64, device=dev)
    table = torch.ones(8, 16, dtype=torch.bfloat16, device=dev)
    out = torch.empty(3, 16, dtype=torch.bfloat16, device=dev)
    hook = _Hook()
    mtb.vocab_embed_fwd(3, 8, 0, 16, mtb.BF16, ids, table, out, comm=hook.comm)
    torch.cuda.synchronize()
    assert hook.calls == [(3 * 16, mtb.BF16, mtb.OP_SUM)]
