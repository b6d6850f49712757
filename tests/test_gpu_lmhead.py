"""GPU parity of the fused LM head + vocab-parallel cross-entropy
(mtb_lmhead_xent_fwd / _bwd) against the fp64 oracle: logits z_r = h W_r^T of
one vocab shard ([TP-block] sec. 4's sharded logits from a column-parallel
output layer), the loss from the three reductions, and the gradients
dh = dz W_r (summed over shards) and dW_r = dz^T h.

Several shards: the R ranks run in R host threads, and the reduction hook
(the all-reduces of sec. 4 and the backward's input-gradient sum) meets the
other threads at a barrier and reduces their buffers with torch. A shard
with no hook is the whole vocabulary, so its targets lie inside it.
"""
import threading

import numpy as np
import pytest
import torch

from gpu_util import TOL, host, rel_err, say
from oracle import lmhead as ol
from transformer_layer_ln_amd import inputs, mtb

pytestmark = pytest.mark.gpu


def _dev_inputs(h, w, target, dloss):
    dev = torch.device("cuda")
    return (torch.as_tensor(h).to(dev, torch.bfloat16).contiguous(),
            torch.as_tensor(w).to(dev, torch.bfloat16).contiguous(),
            torch.as_tensor(target).to(dev), torch.as_tensor(dloss).to(dev, torch.float32))


def _run_one(h, w, target, v0, dloss, comm=None, want=("loss", "dh", "dw"), store=False):
    """One shard through the C ABI -> host dict(loss, stats, dh, dw); store:
    the forward keeps the logits and the backward uses them (no workspace)."""
    n, H = h.shape
    vl = w.shape[0]
    hd, wd, td, dl = _dev_inputs(h, w, target, dloss)
    ws = torch.empty(mtb.lmhead_xent_workspace_bytes(n, H, vl), dtype=torch.uint8, device=hd.device)
    stats = torch.full((4, n), float("nan"), device=hd.device)
    loss = torch.full((n,), float("nan"), device=hd.device) if "loss" in want else None
    z = torch.full((n, vl), float("nan"), dtype=torch.bfloat16, device=hd.device) if store else None
    mtb.lmhead_xent_fwd(n, H, vl, v0, mtb.BF16, hd, wd, td, stats, loss, ws, comm=comm, logits=z)
    zhost = host(z) if store else None
    dh = torch.full_like(hd, float("nan")) if "dh" in want else None
    dw = torch.full_like(wd, float("nan")) if "dw" in want else None
    mtb.lmhead_xent_bwd(n, H, vl, v0, mtb.BF16, hd, wd, td, stats, dl, dh, dw,
                        None if store else ws, comm=comm, logits=z)
    torch.cuda.synchronize()
    out = dict(stats=host(stats))
    if store:
        out["logits"] = zhost
    for k, t in (("loss", loss), ("dh", dh), ("dw", dw)):
        if t is not None:
            out[k] = host(t)
    return out


def _oracle_full(h, w_shards, target, v0s, dloss):
    loss, gmax, sexp, zs = ol.forward(h, w_shards, target, v0s)
    dh = 0.0
    dws = []
    for w, z, a in zip(w_shards, zs, v0s):
        p, dw = ol.backward_shard(h, w, z, target, a, gmax, sexp, dloss)
        dh = dh + p
        dws.append(dw)
    return dict(loss=loss, gmax=gmax, dh=dh, dws=dws)


def _check(got, ref, tag, has_dw=True):
    e_loss = rel_err(got["loss"], ref["loss"])
    e_m = rel_err(got["stats"][0], ref["gmax"])
    e_dh = rel_err(got["dh"], ref["dh"])
    e_dw = rel_err(got["dw"], ref["dws"][0]) if has_dw else 0.0
    say(f"   {tag}: loss {e_loss:.2e}  max {e_m:.2e}  dh {e_dh:.2e}  dW {e_dw:.2e}")
    assert e_loss <= TOL["f32"] and e_m <= TOL["f32"], (e_loss, e_m)
    assert e_dh <= TOL["bf16"] and e_dw <= TOL["bf16"], (e_dh, e_dw)


@pytest.mark.parametrize("n,H,V", [
    (264, 200, 1000),      # ragged against every tile, a partial last k-tile
    (8, 8, 8),             # the smallest legal shape
    (1032, 1032, 2056),
    (520, 4096, 760),      # a full-depth contraction, narrow vocab
    (4096, 64, 16032),     # shallow, the seq-4096 shard's vocab width
])
def test_single_shard_matches_oracle(n, H, V):
    cfg = inputs.LmheadConfig("lmhead-one", n_tokens=n, vocab=V, hidden=H, tp=1, seed=3300 + n,
                              w_std=0.5 / np.sqrt(H))
    say(f"[gpu] LM head, one shard: n={n} hidden={H} vocab={V}")
    h, w = inputs.lmhead_h(cfg), inputs.lmhead_w(cfg, 0)
    t = inputs.lmhead_targets(cfg)
    dloss = np.random.default_rng(7).uniform(0.5, 1.5, n).astype(np.float32) / n
    got = _run_one(h, w, t, 0, dloss)
    _check(got, _oracle_full(h, [w], t, [0], dloss), "one shard")


def test_output_selection_and_determinism():
    cfg = inputs.LmheadConfig("lmhead-sel", n_tokens=136, vocab=1064, hidden=328, tp=1, seed=3400)
    say("[gpu] LM head: loss/dh/dw optional, bitwise repeatable")
    h, w, t = inputs.lmhead_h(cfg), inputs.lmhead_w(cfg, 0), inputs.lmhead_targets(cfg)
    dloss = np.full(136, 1.0 / 136, np.float32)
    a = _run_one(h, w, t, 0, dloss)
    b = _run_one(h, w, t, 0, dloss)
    a["stats"], b["stats"] = a["stats"][:3], b["stats"][:3]   # row 3: scratch of the hook path
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c = _run_one(h, w, t, 0, dloss, want=("dh",))
    d = _run_one(h, w, t, 0, dloss, want=("dw",))
    assert np.array_equal(c["dh"], a["dh"]) and np.array_equal(d["dw"], a["dw"])
    assert np.array_equal(c["stats"][:3], a["stats"][:3])


class _ThreadedAllreduce:
    """R ranks in R host threads: each hook call parks its buffer, the last
    to arrive reduces all R (fp32 arithmetic) and writes the result back."""

    def __init__(self, R):
        self.R = R
        self.bar = threading.Barrier(R, timeout=120)
        self.slots = [None] * R
        self.calls = [[] for _ in range(R)]
        self.local = threading.local()
        self.fn = mtb.ALLREDUCE_FN(self._cb)
        self.comm = mtb.Comm(self.fn, None)

    def bind(self, rank, bufs):
        self.local.rank = rank
        self.local.bufs = bufs

    def _view(self, ptr, count, dtype):
        for t in self.local.bufs:
            off = ptr - t.data_ptr()
            if 0 <= off < t.numel() * t.element_size():
                assert off % t.element_size() == 0
                flat = t.view(-1)
                i = off // t.element_size()
                assert i + count <= flat.numel()
                assert t.dtype == (torch.bfloat16 if dtype == mtb.BF16 else torch.float32)
                return flat[i:i + count]
        raise AssertionError("hook buffer outside the registered tensors")

    def _cb(self, buf, count, dtype, op, stream, user):
        try:
            r = self.local.rank
            self.calls[r].append((count, dtype, op))
            torch.cuda.synchronize()
            self.slots[r] = (self._view(buf, count, dtype), op)
            if self.bar.wait() == 0:
                views = [s[0] for s in self.slots]
                assert all(s[1] == op for s in self.slots)
                acc = torch.stack([v.float() for v in views])
                res = acc.max(0).values if op == mtb.OP_MAX else acc.sum(0)
                for v in views:
                    v.copy_(res.to(v.dtype))
                torch.cuda.synchronize()
            self.bar.wait()
            return 0
        except Exception as e:   # noqa: BLE001 -- reported by the calling thread
            self.bar.abort()
            print("hook error:", e, flush=True)
            return 1


def _run_threaded(cfg, h, w_shards, target, dloss):
    R = cfg.tp
    ar = _ThreadedAllreduce(R)
    n, H = h.shape
    vl = cfg.v_local
    res = [None] * R
    err = []

    def rank(r):
        try:
            hd, wd, td, dl = _dev_inputs(h, w_shards[r], target, dloss)
            stats = torch.full((4, n), float("nan"), device=hd.device)
            loss = torch.full((n,), float("nan"), device=hd.device)
            dh = torch.full_like(hd, float("nan"))
            dw = torch.full_like(wd, float("nan"))
            ws = torch.empty(mtb.lmhead_xent_workspace_bytes(n, H, vl), dtype=torch.uint8,
                             device=hd.device)
            torch.cuda.synchronize()
            ar.bind(r, [stats, dh])
            mtb.lmhead_xent_fwd(n, H, vl, r * vl, mtb.BF16, hd, wd, td, stats, loss, ws,
                                comm=ar.comm)
            mtb.lmhead_xent_bwd(n, H, vl, r * vl, mtb.BF16, hd, wd, td, stats, dl, dh, dw, ws,
                                comm=ar.comm)
            torch.cuda.synchronize()
            res[r] = dict(loss=host(loss), stats=host(stats), dh=host(dh), dw=host(dw))
        except Exception as e:   # noqa: BLE001
            err.append((r, e))
            ar.bar.abort()

    ths = [threading.Thread(target=rank, args=(r,)) for r in range(R)]
    for t in ths:
        t.start()
    for t in ths:
        t.join(300)
    assert not err, err
    assert all(not t.is_alive() for t in ths)
    return res, ar.calls


@pytest.mark.parametrize("n,H,V,R", [(264, 200, 4000, 4), (1024, 512, 8 * 1032, 8)])
def test_vocab_shards_with_reduction_hook(n, H, V, R):
    cfg = inputs.LmheadConfig("lmhead-tp", n_tokens=n, vocab=V, hidden=H, tp=R, seed=3500 + R,
                              w_std=1.0 / np.sqrt(H))
    say(f"[gpu] LM head, {R} vocab shards in threads: n={n} hidden={H} vocab={V}")
    h, t = inputs.lmhead_h(cfg), inputs.lmhead_targets(cfg)
    ws = [inputs.lmhead_w(cfg, r) for r in range(R)]
    dloss = np.full(n, 1.0 / n, np.float32)
    res, calls = _run_threaded(cfg, h, ws, t, dloss)
    for r in range(R):
        assert calls[r] == [(n, mtb.F32, mtb.OP_MAX), (n, mtb.F32, mtb.OP_SUM),
                            (n, mtb.F32, mtb.OP_SUM), (n * H, mtb.BF16, mtb.OP_SUM)], calls[r]
    ref = _oracle_full(h, ws, t, [r * cfg.v_local for r in range(R)], dloss)
    for r in range(R):
        got = res[r]
        assert np.array_equal(got["loss"], res[0]["loss"]) and np.array_equal(got["dh"], res[0]["dh"])
        _check(dict(got, dw=got["dw"]), dict(ref, dws=[ref["dws"][r]]), f"shard {r}")


def test_seq4096_vocab_shard_full_size():
    """One [8192 tokens x 4096] x [16032 x 4096] shard of the vocab-128256
    output layer (the launch bench.py times), no hook: the shard is the whole
    vocabulary, so targets are drawn inside it. Loss and max on every token,
    dh on sampled tokens, dW on three vocab-row ranges (first, middle, the
    ragged last tile); the oracle runs over all tokens in row chunks."""
    cfg = inputs.C5_LMHEAD
    r = cfg.tp - 1
    v0 = r * cfg.v_local
    say(f"[gpu] LM head {cfg.name}, shard {r}, full size")
    h, w = inputs.lmhead_h(cfg), inputs.lmhead_w(cfg, r)
    t = v0 + inputs.lmhead_targets(cfg) % cfg.v_local
    n = cfg.n_tokens
    dloss = np.full(n, 1.0 / n, np.float32)
    got = _run_one(h, w, t, v0, dloss)
    rows = np.unique(np.concatenate([np.arange(0, n, 131), np.arange(n - 9, n)]))
    vr = cfg.v_local
    cols = [(0, 64), (vr // 2, vr // 2 + 64), (vr - 96, vr)]
    ref_loss = np.empty(n)
    ref_m = np.empty(n)
    ref_dh = {}
    ref_dw = [0.0] * len(cols)
    CH = 1024
    for c0 in range(0, n, CH):
        sl = slice(c0, min(n, c0 + CH))
        loss, gmax, sexp, zs = ol.forward(h[sl], [w], t[sl], [v0])
        ref_loss[sl], ref_m[sl] = loss, gmax
        sel = rows[(rows >= sl.start) & (rows < sl.stop)]
        if sel.size:
            i = sel - c0
            p, _ = ol.backward_shard(h[sel], w, zs[0][i], t[sel], v0, gmax[i], sexp[i], dloss[sel])
            for k, s in enumerate(sel):
                ref_dh[s] = p[k]
        for k, (a, b) in enumerate(cols):
            _, dw = ol.backward_shard(h[sl], w[a:b], zs[0][:, a:b], t[sl], v0 + a, gmax, sexp,
                                      dloss[sl])
            ref_dw[k] = ref_dw[k] + dw
    e = [rel_err(got["loss"], ref_loss), rel_err(got["stats"][0], ref_m),
         rel_err(got["dh"][rows], np.stack([ref_dh[s] for s in rows]))]
    e += [rel_err(got["dw"][a:b], ref_dw[k]) for k, (a, b) in enumerate(cols)]
    say(f"   loss {e[0]:.2e}  max {e[1]:.2e}  dh {e[2]:.2e}  dW " + " ".join(f"{x:.2e}" for x in e[3:]))
    assert e[0] <= TOL["f32"] and e[1] <= TOL["f32"]
    assert max(e[2:]) <= TOL["bf16"]
    assert np.all(np.isfinite(got["dh"])) and np.all(np.isfinite(got["dw"]))


@pytest.mark.parametrize("n,H,V", [(264, 200, 1000), (1032, 1032, 2056)])
def test_stored_logits_mode(n, H, V):
    """Logits kept by the forward (bf16) and used by the backward in place of
    the recompute: the stored logits are the product rounded once, the loss
    is that of the stored logits (bf16-level agreement with the fp64 oracle),
    and the gradients match the oracle and the recompute path."""
    cfg = inputs.LmheadConfig("lmhead-store", n_tokens=n, vocab=V, hidden=H, tp=1, seed=3600 + n,
                              w_std=0.5 / np.sqrt(H))
    say(f"[gpu] LM head, stored logits: n={n} hidden={H} vocab={V}")
    h, w, t = inputs.lmhead_h(cfg), inputs.lmhead_w(cfg, 0), inputs.lmhead_targets(cfg)
    dloss = np.full(n, 1.0 / n, np.float32)
    got = _run_one(h, w, t, 0, dloss, store=True)
    ref = _oracle_full(h, [w], t, [0], dloss)
    z_ref = ol.logits(h, w)
    assert rel_err(got["logits"], z_ref) <= TOL["bf16"]
    e = {k: rel_err(got[k], ref[k]) for k in ("loss", "dh")}
    e["dW"] = rel_err(got["dw"], ref["dws"][0])
    say("   " + "  ".join(f"{k} {v:.2e}" for k, v in e.items()))
    assert max(e.values()) <= TOL["bf16"]
    rec = _run_one(h, w, t, 0, dloss)
    assert rel_err(got["dh"], rec["dh"]) <= 1e-2 and rel_err(got["dw"], rec["dw"]) <= 1e-2
