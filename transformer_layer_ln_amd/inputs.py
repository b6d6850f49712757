"""Seeded synthetic inputs for the tensor-parallel Transformer block and the
vocab-sharded cross-entropy.

This module is shared by the tests, the benchmark and the oracle checks. It
holds shapes, random draws and bf16 rounding only: none of the block's
arithmetic lives here.

Recipe (every tensor is its own counter-keyed stream, so one rank's shard can
be drawn without drawing the others, and the unsharded tensor is the
concatenation of all shards' draws):

* generator: ``numpy.random.default_rng([seed, tag, shard])`` (PCG64 seeded
  through SeedSequence), ``seed = 1000 + config number``;
* activations ``x`` and the parity cotangent ``G`` ~ N(0, 1), shape [B, S, H];
* weights ~ N(0, 1/fan_in) with fan_in the *unsharded* input dimension
  (H for QKV and fc1, q_heads_full * head_dim for the output projection,
  ffn_full for fc2);
* optional biases ~ N(0, 1/fan_in), optional LayerNorm gain ~ 1 + 0.1 N(0,1)
  and shift ~ 0.1 N(0,1) (only the affine/bias parity variant uses them);
* vocab logits ~ N(0, 1) per vocab shard [N, V_local], targets uniform
  integers in [0, V);
* draws are float32; bf16 configurations round them to bf16 by
  round-to-nearest-even and keep the rounded values in float32 arrays, so
  every consumer sees exactly the same numbers.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

import numpy as np

# stream tags: one per drawn tensor
_TAG = {
    "x": 1, "g": 2,
    "wq": 10, "wk": 11, "wv": 12, "wo": 13, "w1": 14, "wg": 15, "wu": 16, "w2": 17,
    "bq": 20, "bk": 21, "bv": 22, "bo": 23, "b1": 24, "bg": 25, "bu": 26, "b2": 27,
    "ln1_g": 30, "ln1_b": 31, "ln2_g": 32, "ln2_b": 33,
    "logits": 40, "targets": 41,
    "embed_table": 50, "embed_ids": 51, "embed_dout": 52,
    "lmhead_h": 60, "lmhead_w": 61, "lmhead_targets": 62,
}


@dataclass(frozen=True)
class BlockConfig:
    """One tensor-parallel rank's share of a Transformer block.

    ``q_heads``, ``kv_heads`` and ``ffn`` are the LOCAL (per-rank) sizes;
    the unsharded layer has ``tp`` times as many.
    """
    name: str
    batch: int
    seq: int
    hidden: int
    q_heads: int
    kv_heads: int
    head_dim: int
    ffn: int
    act: str = "gelu"          # "gelu" | "swiglu"
    causal: bool = False
    dtype: str = "bf16"        # "f32" | "bf16"
    tp: int = 1
    seed: int = 1000
    affine: bool = False       # LayerNorm gain/shift present
    bias: bool = False         # linear biases present
    ln_eps: float = 1e-5
    norm: str = "pre"          # "pre" | "post": LayerNorm before each sublayer or after each residual
    p_attn: float = 0.0        # dropout on the attention probabilities
    p_hidden: float = 0.0      # dropout on the hidden state after attention and after the MLP
    drop_seed: int = 0
    drop_offset: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    @property
    def n_qkv(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim

    def full(self) -> "BlockConfig":
        """The unsharded layer (tp = 1) this rank's share belongs to."""
        return dataclasses.replace(self, q_heads=self.q_heads * self.tp,
                                   kv_heads=self.kv_heads * self.tp,
                                   ffn=self.ffn * self.tp, tp=1)

    def with_(self, **kw) -> "BlockConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class XentConfig:
    name: str
    n_tokens: int
    vocab: int
    tp: int
    dtype: str = "bf16"
    seed: int = 1005

    @property
    def v_local(self) -> int:
        return self.vocab // self.tp


@dataclass(frozen=True)
class EmbedConfig:
    """Vocab-parallel input embedding: a [vocab, hidden] table split by vocab
    over tp ranks; n_tokens token ids. repeat > 0 draws the ids from only
    `repeat` distinct values (heavy rows for the scatter-add)."""
    name: str
    n_tokens: int
    vocab: int
    hidden: int
    tp: int
    dtype: str = "bf16"
    seed: int = 1005
    repeat: int = 0

    @property
    def v_local(self) -> int:
        return self.vocab // self.tp


@dataclass(frozen=True)
class LmheadConfig:
    """Vocab-parallel output layer + cross-entropy: final hidden states
    [n_tokens, hidden] (N(0,1), what a LayerNorm with unit gain hands over),
    a [vocab, hidden] output embedding split by vocab over tp ranks (N(0,
    w_std^2), the usual 0.02 initialisation), uniform targets in [0, vocab)."""
    name: str
    n_tokens: int
    vocab: int
    hidden: int
    tp: int
    seed: int = 1006
    w_std: float = 0.02

    @property
    def v_local(self) -> int:
        return self.vocab // self.tp


# The five workloads. C1 is the small fp32 correctness case; C2-C5 are one
# rank's share of the tensor-parallel layers the pages describe.
C1 = BlockConfig("C1-fp32-full", batch=1, seq=64, hidden=128, q_heads=4, kv_heads=4,
                 head_dim=32, ffn=512, act="gelu", causal=False, dtype="f32", tp=1, seed=1001)
C2 = BlockConfig("C2-tp4-s512", batch=8, seq=512, hidden=1024, q_heads=4, kv_heads=4,
                 head_dim=64, ffn=1024, act="gelu", causal=False, dtype="bf16", tp=4, seed=1002)
C3_SEQS = (128, 256, 512, 1024)


def C3(seq: int) -> BlockConfig:
    return C2.with_(name=f"C3-tp4-s{seq}", seq=seq, seed=1003)


C4 = BlockConfig("C4-tp8-s2048-causal", batch=4, seq=2048, hidden=4096, q_heads=4, kv_heads=4,
                 head_dim=128, ffn=2048, act="gelu", causal=True, dtype="bf16", tp=8, seed=1004)
C5 = BlockConfig("C5-tp8-s4096-swiglu-gqa", batch=2, seq=4096, hidden=4096, q_heads=4, kv_heads=1,
                 head_dim=128, ffn=1792, act="swiglu", causal=False, dtype="bf16", tp=8, seed=1005)
C5_XENT = XentConfig("C5-xent-v128256-tp8", n_tokens=8192, vocab=128256, tp=8, dtype="bf16", seed=1005)
# the input-side counterpart of C5's vocab shard: ids of the seq-4096 share's
# 8192 tokens, one [16032 x 4096] shard of the 128256-row table
C5_EMBED = EmbedConfig("C5-embed-v128256-h4096-tp8", n_tokens=8192, vocab=128256, hidden=4096, tp=8)
# the output layer of the same model: the seq-4096 share's final hidden
# states against one vocab shard of the [128256, 4096] output embedding
C5_LMHEAD = LmheadConfig("C5-lmhead-v128256-h4096-tp8", n_tokens=8192, vocab=128256, hidden=4096,
                         tp=8)

CONFIGS = {"C1": C1, "C2": C2, "C4": C4, "C5": C5}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(seed: int, name: str, shard: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, _TAG[name], shard])


def _normal(seed, name, shard, shape, std, dtype):
    a = _rng(seed, name, shard).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_bf16(a) if dtype == "bf16" else a


def _affine(seed, name, shard, shape, base, scale, dtype):
    a = _rng(seed, name, shard).standard_normal(shape, dtype=np.float32) * np.float32(scale)
    a += np.float32(base)
    return round_bf16(a) if dtype == "bf16" else a


def activations(cfg: BlockConfig) -> dict:
    """x and the parity cotangent G, both [B, S, H] (replicated over ranks)."""
    shp = (cfg.batch, cfg.seq, cfg.hidden)
    return {"x": _normal(cfg.seed, "x", 0, shp, 1.0, cfg.dtype),
            "g": _normal(cfg.seed, "g", 0, shp, 1.0, cfg.dtype)}


def shard_weights(cfg: BlockConfig, rank: int = 0) -> dict:
    """Rank ``rank``'s weights, in the [out, in] orientation, split apart:
    wq [nq*d, H], wk/wv [nkv*d, H], wo [H, nq*d], w1 [F, H] (GELU) or
    wg/wu [F, H] (SwiGLU), w2 [H, F]; plus optional biases and LN gain/shift.
    Row-parallel biases (bo, b2) and LN parameters are replicated (drawn with
    shard 0 for every rank)."""
    H, d, nq, nkv, F = cfg.hidden, cfg.head_dim, cfg.q_heads, cfg.kv_heads, cfg.ffn
    s, dt = cfg.seed, cfg.dtype
    std_h = 1.0 / np.sqrt(H)
    std_o = 1.0 / np.sqrt(nq * cfg.tp * d)
    std_2 = 1.0 / np.sqrt(F * cfg.tp)
    w = {"wq": _normal(s, "wq", rank, (nq * d, H), std_h, dt),
         "wk": _normal(s, "wk", rank, (nkv * d, H), std_h, dt),
         "wv": _normal(s, "wv", rank, (nkv * d, H), std_h, dt),
         "wo": _normal(s, "wo", rank, (H, nq * d), std_o, dt),
         "w2": _normal(s, "w2", rank, (H, F), std_2, dt)}
    if cfg.act == "gelu":
        w["w1"] = _normal(s, "w1", rank, (F, H), std_h, dt)
    else:
        w["wg"] = _normal(s, "wg", rank, (F, H), std_h, dt)
        w["wu"] = _normal(s, "wu", rank, (F, H), std_h, dt)
    if cfg.bias:
        w["bq"] = _normal(s, "bq", rank, (nq * d,), std_h, dt)
        w["bk"] = _normal(s, "bk", rank, (nkv * d,), std_h, dt)
        w["bv"] = _normal(s, "bv", rank, (nkv * d,), std_h, dt)
        w["bo"] = _normal(s, "bo", 0, (H,), std_o, dt)
        w["b2"] = _normal(s, "b2", 0, (H,), std_2, dt)
        if cfg.act == "gelu":
            w["b1"] = _normal(s, "b1", rank, (F,), std_h, dt)
        else:
            w["bg"] = _normal(s, "bg", rank, (F,), std_h, dt)
            w["bu"] = _normal(s, "bu", rank, (F,), std_h, dt)
    if cfg.affine:
        w["ln1_g"] = _affine(s, "ln1_g", 0, (H,), 1.0, 0.1, dt)
        w["ln1_b"] = _affine(s, "ln1_b", 0, (H,), 0.0, 0.1, dt)
        w["ln2_g"] = _affine(s, "ln2_g", 0, (H,), 1.0, 0.1, dt)
        w["ln2_b"] = _affine(s, "ln2_b", 0, (H,), 0.0, 0.1, dt)
    return w


_COL = ("wq", "wk", "wv", "w1", "wg", "wu", "bq", "bk", "bv", "b1", "bg", "bu")   # split on dim 0
_ROW = ("wo", "w2")                                                         # split on dim 1
_REP = ("bo", "b2", "ln1_g", "ln1_b", "ln2_g", "ln2_b")                     # replicated


def full_weights(cfg: BlockConfig) -> dict:
    """The unsharded layer: every rank's shard concatenated in rank order."""
    shards = [shard_weights(cfg, r) for r in range(cfg.tp)]
    out = {}
    for k in shards[0]:
        if k in _COL:
            out[k] = np.concatenate([sh[k] for sh in shards], axis=0)
        elif k in _ROW:
            out[k] = np.concatenate([sh[k] for sh in shards], axis=1)
        else:
            out[k] = shards[0][k]
    return out


def xent_logits(cfg: XentConfig, rank: int, rows: slice | None = None) -> np.ndarray:
    """Vocab shard ``rank``'s logits [N, V_local] (float32, bf16-exact for bf16)."""
    z = _normal(cfg.seed, "logits", rank, (cfg.n_tokens, cfg.v_local), 1.0, cfg.dtype)
    return z if rows is None else z[rows]


def xent_targets(cfg: XentConfig) -> np.ndarray:
    return _rng(cfg.seed, "targets").integers(0, cfg.vocab, size=cfg.n_tokens, dtype=np.int64)


def xent_dloss(cfg: XentConfig) -> np.ndarray:
    """Per-token loss cotangent for a mean over tokens: 1/N each (float32)."""
    return np.full(cfg.n_tokens, 1.0 / cfg.n_tokens, dtype=np.float32)


def embed_table(cfg: EmbedConfig, rank: int) -> np.ndarray:
    """Vocab shard ``rank``'s table rows [V_local, hidden], N(0,1)."""
    return _normal(cfg.seed, "embed_table", rank, (cfg.v_local, cfg.hidden), 1.0, cfg.dtype)


def embed_ids(cfg: EmbedConfig) -> np.ndarray:
    """Token ids [N] int64, uniform in [0, vocab) (or over `repeat` values)."""
    r = _rng(cfg.seed, "embed_ids")
    if cfg.repeat:
        pool = r.integers(0, cfg.vocab, size=cfg.repeat, dtype=np.int64)
        return pool[r.integers(0, cfg.repeat, size=cfg.n_tokens)]
    return r.integers(0, cfg.vocab, size=cfg.n_tokens, dtype=np.int64)


def embed_dout(cfg: EmbedConfig) -> np.ndarray:
    """Gradient of the embedding output [N, hidden], N(0,1)."""
    return _normal(cfg.seed, "embed_dout", 0, (cfg.n_tokens, cfg.hidden), 1.0, cfg.dtype)


def lmhead_h(cfg: LmheadConfig) -> np.ndarray:
    """Final hidden states [N, hidden] (bf16-exact float32)."""
    return _normal(cfg.seed, "lmhead_h", 0, (cfg.n_tokens, cfg.hidden), 1.0, "bf16")


def lmhead_w(cfg: LmheadConfig, rank: int) -> np.ndarray:
    """Vocab shard ``rank``'s output-embedding rows [V_local, hidden]."""
    return _normal(cfg.seed, "lmhead_w", rank, (cfg.v_local, cfg.hidden), cfg.w_std, "bf16")


def lmhead_targets(cfg: LmheadConfig) -> np.ndarray:
    return _rng(cfg.seed, "lmhead_targets").integers(0, cfg.vocab, size=cfg.n_tokens,
                                                     dtype=np.int64)
