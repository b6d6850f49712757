"""Thin ctypes binding of libmtb (see include/mtb.h for the contract).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the block runs in libmtb's kernels. There
is no fallback: if the library is missing or the call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmtb.so")

MTB_OK, MTB_EINVAL, MTB_EUNSUPPORTED, MTB_EHIP, MTB_ECOMM = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ACT_GELU, ACT_SWIGLU = 0, 1
NORM_PRE, NORM_POST = 0, 1
OP_SUM, OP_MAX = 0, 1
PHASE_ALL, PHASE_SEG0, PHASE_SEG1, PHASE_SEG2 = 0, 1, 2, 3
XENT_PARTIAL, XENT_FINISH, XENT_ALL = 0, 1, 2

WEIGHT_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                 "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")

# the functions include/mtb.h declares
EXPORTS = ("mtb_block_saved_bytes", "mtb_block_scratch_bytes", "mtb_block_fwd", "mtb_block_bwd",
           "mtb_vocab_xent", "mtb_vocab_xent_combine", "mtb_lmhead_xent_workspace_bytes",
           "mtb_lmhead_xent_fwd", "mtb_lmhead_xent_bwd", "mtb_vocab_embed_fwd",
           "mtb_vocab_embed_bwd_workspace_bytes", "mtb_vocab_embed_bwd",
           "mtb_vocab_embed_bwd_noalloc", "mtb_trace_arm",
           "mtb_trace_disarm", "mtb_last_error")
TRACE_NONE, TRACE_FC1_FWD, TRACE_ATTN_FWD, TRACE_LN1_FWD, TRACE_FC2_WGRAD = 0, 1, 2, 3, 4
TRACE_ATTN_SEG, TRACE_FFN_SEG, TRACE_BWD, TRACE_LN1_BWD = 5, 6, 7, 8


class MtbError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libmtb status {status}: {msg}")
        self.status = status


class Cfg(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("seq", c_int32), ("hidden", c_int32),
                ("q_heads", c_int32), ("kv_heads", c_int32), ("head_dim", c_int32),
                ("ffn", c_int32), ("act", c_int32), ("causal", c_int32), ("dtype", c_int32),
                ("ln_eps", c_float), ("norm", c_int32), ("attn_dropout", c_float),
                ("hidden_dropout", c_float), ("tp_rank", c_int32), ("rng_offset", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]


class Weights(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in WEIGHT_FIELDS]


class Grads(ctypes.Structure):
    _fields_ = [(f, c_void_p) for f in WEIGHT_FIELDS]


ALLREDUCE_FN = ctypes.CFUNCTYPE(c_int32, c_void_p, c_int64, c_int32, c_int32, c_void_p, c_void_p)


class Comm(ctypes.Structure):
    _fields_ = [("allreduce", ALLREDUCE_FN), ("user", c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmtb.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m transformer_layer_ln_amd.build`")
    lib = ctypes.CDLL(path)
    lib.mtb_block_saved_bytes.argtypes = [POINTER(Cfg)]
    lib.mtb_block_saved_bytes.restype = c_size_t
    lib.mtb_block_scratch_bytes.argtypes = [POINTER(Cfg)]
    lib.mtb_block_scratch_bytes.restype = c_size_t
    lib.mtb_block_fwd.argtypes = [POINTER(Cfg), POINTER(Weights), c_int32, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, POINTER(Comm), c_void_p]
    lib.mtb_block_fwd.restype = c_int32
    lib.mtb_block_bwd.argtypes = [POINTER(Cfg), POINTER(Weights), c_int32, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, POINTER(Grads), c_void_p,
                                  POINTER(Comm), c_void_p]
    lib.mtb_block_bwd.restype = c_int32
    lib.mtb_vocab_xent.argtypes = [c_int64, c_int64, c_int64, c_int32, c_int32, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   POINTER(Comm), c_void_p]
    lib.mtb_vocab_xent.restype = c_int32
    lib.mtb_vocab_xent_combine.argtypes = [c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.mtb_vocab_xent_combine.restype = c_int32
    lib.mtb_lmhead_xent_workspace_bytes.argtypes = [c_int64, c_int64, c_int64]
    lib.mtb_lmhead_xent_workspace_bytes.restype = c_size_t
    lib.mtb_lmhead_xent_fwd.argtypes = [c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p]
    lib.mtb_lmhead_xent_fwd.restype = c_int32
    lib.mtb_lmhead_xent_bwd.argtypes = [c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p]
    lib.mtb_lmhead_xent_bwd.restype = c_int32
    lib.mtb_vocab_embed_fwd.argtypes = [c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p]
    lib.mtb_vocab_embed_fwd.restype = c_int32
    lib.mtb_vocab_embed_bwd_workspace_bytes.argtypes = [c_int64, c_int64]
    lib.mtb_vocab_embed_bwd_workspace_bytes.restype = c_size_t
    lib.mtb_vocab_embed_bwd.argtypes = [c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p]
    lib.mtb_vocab_embed_bwd.restype = c_int32
    lib.mtb_vocab_embed_bwd_noalloc.argtypes = [c_int64, c_int64, c_int64, c_int64, c_int32, c_void_p,
                                                c_void_p, c_void_p, c_void_p]
    lib.mtb_vocab_embed_bwd_noalloc.restype = c_int32
    lib.mtb_trace_arm.argtypes = [c_int32, c_void_p, c_void_p, c_int32]
    lib.mtb_trace_arm.restype = c_int32
    lib.mtb_trace_disarm.argtypes = []
    lib.mtb_trace_disarm.restype = c_int32
    lib.mtb_last_error.argtypes = []
    lib.mtb_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().mtb_last_error().decode()


def _check(status):
    if status != MTB_OK:
        raise MtbError(status, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_cfg(batch, seq, hidden, q_heads, kv_heads, head_dim, ffn, act="gelu", causal=False,
             dtype="bf16", ln_eps=1e-5, norm="pre", attn_dropout=0.0, hidden_dropout=0.0,
             tp_rank=0, rng_offset=0, seed=0) -> Cfg:
    return Cfg(batch, seq, hidden, q_heads, kv_heads, head_dim, ffn,
               ACT_GELU if act == "gelu" else ACT_SWIGLU, int(bool(causal)),
               BF16 if dtype == "bf16" else F32, ln_eps, NORM_POST if norm == "post" else NORM_PRE,
               attn_dropout, hidden_dropout, tp_rank, rng_offset, seed)


def cfg_from(c, tp_rank=0) -> Cfg:
    """Cfg from an object with the BlockConfig attribute names (tp_rank: the
    rank whose share this is, for the attention dropout stream)."""
    return make_cfg(c.batch, c.seq, c.hidden, c.q_heads, c.kv_heads, c.head_dim, c.ffn,
                    c.act, c.causal, c.dtype, c.ln_eps, getattr(c, "norm", "pre"),
                    getattr(c, "p_attn", 0.0), getattr(c, "p_hidden", 0.0), tp_rank,
                    getattr(c, "drop_offset", 0), getattr(c, "drop_seed", 0))


def saved_bytes(cfg: Cfg) -> int:
    return load().mtb_block_saved_bytes(byref(cfg))


def scratch_bytes(cfg: Cfg) -> int:
    return load().mtb_block_scratch_bytes(byref(cfg))


def _weights(w: dict) -> Weights:
    return Weights(*[_ptr(w.get(f)) for f in WEIGHT_FIELDS])


def _grads(g: dict | None) -> Grads | None:
    if g is None:
        return None
    return Grads(*[_ptr(g.get(f)) for f in WEIGHT_FIELDS])


def block_fwd(cfg: Cfg, w: dict, phase, x, reduced_in, out, saved, scratch, comm=None, stream=None):
    _check(load().mtb_block_fwd(byref(cfg), byref(_weights(w)), phase, _ptr(x), _ptr(reduced_in),
                                _ptr(out), _ptr(saved), _ptr(scratch),
                                byref(comm) if comm is not None else None, _stream(stream)))


def block_bwd(cfg: Cfg, w: dict, phase, x, saved, dout, reduced_in, dx, grads: dict | None,
              scratch, comm=None, stream=None):
    g = _grads(grads)
    _check(load().mtb_block_bwd(byref(cfg), byref(_weights(w)), phase, _ptr(x), _ptr(saved),
                                _ptr(dout), _ptr(reduced_in), _ptr(dx),
                                byref(g) if g is not None else None, _ptr(scratch),
                                byref(comm) if comm is not None else None, _stream(stream)))


def vocab_xent(n_tokens, v_local, v_start, dtype, phase, logits, target, stats, loss=None,
               dloss=None, dlogits=None, comm=None, stream=None):
    _check(load().mtb_vocab_xent(n_tokens, v_local, v_start, dtype, phase, _ptr(logits),
                                 _ptr(target), _ptr(stats), _ptr(loss), _ptr(dloss),
                                 _ptr(dlogits), byref(comm) if comm is not None else None,
                                 _stream(stream)))


def vocab_xent_combine(n_tokens, n_shards, shard_stats, stats, loss=None, stream=None):
    _check(load().mtb_vocab_xent_combine(n_tokens, n_shards, _ptr(shard_stats), _ptr(stats),
                                         _ptr(loss), _stream(stream)))


def lmhead_xent_workspace_bytes(n_tokens, hidden, v_local):
    return load().mtb_lmhead_xent_workspace_bytes(n_tokens, hidden, v_local)


def lmhead_xent_fwd(n_tokens, hidden, v_local, v_start, dtype, h, w, target, stats, loss,
                    workspace, comm=None, stream=None, logits=None):
    _check(load().mtb_lmhead_xent_fwd(n_tokens, hidden, v_local, v_start, dtype, _ptr(h), _ptr(w),
                                      _ptr(target), _ptr(stats), _ptr(loss), _ptr(logits),
                                      _ptr(workspace), byref(comm) if comm is not None else None,
                                      _stream(stream)))


def lmhead_xent_bwd(n_tokens, hidden, v_local, v_start, dtype, h, w, target, stats, dloss, dh, dw,
                    workspace, comm=None, stream=None, logits=None):
    _check(load().mtb_lmhead_xent_bwd(n_tokens, hidden, v_local, v_start, dtype, _ptr(h), _ptr(w),
                                      _ptr(target), _ptr(stats), _ptr(dloss), _ptr(logits), _ptr(dh),
                                      _ptr(dw), _ptr(workspace),
                                      byref(comm) if comm is not None else None, _stream(stream)))


def vocab_embed_fwd(n_tokens, v_local, v_start, hidden, dtype, ids, table, out, comm=None,
                    stream=None):
    _check(load().mtb_vocab_embed_fwd(n_tokens, v_local, v_start, hidden, dtype, _ptr(ids),
                                      _ptr(table), _ptr(out),
                                      byref(comm) if comm is not None else None, _stream(stream)))


def vocab_embed_bwd_workspace_bytes(n_tokens, v_local):
    return load().mtb_vocab_embed_bwd_workspace_bytes(n_tokens, v_local)


def vocab_embed_bwd(n_tokens, v_local, v_start, hidden, dtype, ids, dout, dtable, workspace,
                    stream=None):
    _check(load().mtb_vocab_embed_bwd(n_tokens, v_local, v_start, hidden, dtype, _ptr(ids),
                                      _ptr(dout), _ptr(dtable), _ptr(workspace), _stream(stream)))


EMBED_NOALLOC_MAX_ROWS = 262144


def vocab_embed_bwd_noalloc(n_tokens, v_local, v_start, hidden, dtype, ids, dout, dtable,
                            stream=None):
    _check(load().mtb_vocab_embed_bwd_noalloc(n_tokens, v_local, v_start, hidden, dtype, _ptr(ids),
                                              _ptr(dout), _ptr(dtable), _stream(stream)))


class Trace:
    """Arm the library's event trace around one kernel class; the pairs are
    torch.cuda.Events so their elapsed times can be read with torch."""

    def __init__(self, what, n, stream=None):
        import torch
        self.what, self.n = what, n
        st = torch.cuda.current_stream() if stream is None else stream
        self.begin = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        self.end = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.begin + self.end:      # create the underlying hipEvents
            e.record(st)
        torch.cuda.synchronize()
        self._b = (c_void_p * n)(*[e.cuda_event for e in self.begin])
        self._e = (c_void_p * n)(*[e.cuda_event for e in self.end])
        self.count = 0

    def __enter__(self):
        _check(load().mtb_trace_arm(self.what, self._b, self._e, self.n))
        return self

    def __exit__(self, *exc):
        self.count = load().mtb_trace_disarm()
        return False

    def mean_ms(self):
        import torch
        torch.cuda.synchronize()
        t = [self.begin[i].elapsed_time(self.end[i]) for i in range(self.count)]
        return sum(t) / len(t) if t else float("nan")


# ---------------------------------------------------------------------------
# layout helpers (pure data movement) and a per-rank convenience wrapper
# ---------------------------------------------------------------------------
def interleave_gate_up(g, u):
    """[F, ...] gate and up rows -> [2F, ...] in blocks of 16 (gate block, up block)."""
    import torch
    F = g.shape[0]
    rest = tuple(g.shape[1:])
    return torch.stack([g.reshape(F // 16, 16, *rest), u.reshape(F // 16, 16, *rest)], 1).reshape(2 * F, *rest)


def split_gate_up(w):
    """Inverse of interleave_gate_up."""
    F2 = w.shape[0]
    rest = tuple(w.shape[1:])
    v = w.reshape(F2 // 32, 2, 16, *rest)
    return v[:, 0].reshape(F2 // 2, *rest), v[:, 1].reshape(F2 // 2, *rest)


def device_weights(w: dict, act: str, dtype, device) -> dict:
    """ABI weight tensors from the split arrays (wq, wk, wv, wo, w1 | wg, wu, w2, biases, LN)."""
    import numpy as np
    import torch
    t = lambda a: torch.as_tensor(a).to(device=device, dtype=dtype).contiguous()
    out = {"w_qkv": t(np.concatenate([w["wq"], w["wk"], w["wv"]], 0)),
           "w_o": t(w["wo"]), "w_fc2": t(w["w2"])}
    if act == "gelu":
        out["w_fc1"] = t(w["w1"])
    else:
        out["w_fc1"] = interleave_gate_up(t(w["wg"]), t(w["wu"])).contiguous()
    if "bq" in w:
        out["b_qkv"] = t(np.concatenate([w["bq"], w["bk"], w["bv"]], 0))
        out["b_o"] = t(w["bo"])
        out["b_fc2"] = t(w["b2"])
        out["b_fc1"] = t(w["b1"]) if act == "gelu" else interleave_gate_up(t(w["bg"]), t(w["bu"])).contiguous()
    for k in ("ln1_g", "ln1_b", "ln2_g", "ln2_b"):
        if k in w:
            out[k] = t(w[k])
    return out


class BlockShard:
    """One rank's share: owns its saved/scratch buffers (torch allocations)."""

    def __init__(self, cfg: Cfg, weights: dict, device="cuda"):
        import torch
        self.cfg = cfg
        self.w = weights
        self.dtype = torch.bfloat16 if cfg.dtype == BF16 else torch.float32
        self.saved = torch.empty(saved_bytes(cfg), dtype=torch.uint8, device=device)
        self.scratch = torch.empty(scratch_bytes(cfg), dtype=torch.uint8, device=device)
        if self.saved.numel() == 0:
            raise MtbError(MTB_EINVAL, last_error())

    def fwd(self, x, out, phase=PHASE_ALL, reduced_in=None, comm=None, stream=None):
        block_fwd(self.cfg, self.w, phase, x, reduced_in, out, self.saved, self.scratch, comm, stream)

    def bwd(self, x, dout, dx, grads=None, phase=PHASE_ALL, reduced_in=None, comm=None, stream=None):
        block_bwd(self.cfg, self.w, phase, x, self.saved, dout, reduced_in, dx, grads, self.scratch,
                  comm, stream)

    def grad_buffers(self, names=None) -> dict:
        import torch
        names = names or [k for k in WEIGHT_FIELDS if k in self.w]
        return {k: torch.empty_like(self.w[k]) for k in names}
