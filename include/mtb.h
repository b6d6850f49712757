/*
 * mtb.h -- C ABI of libmtb: forward and backward of one tensor-parallel
 * rank's share of a Megatron-style Transformer block, and the vocab-sharded
 * cross-entropy, on one AMD Instinct MI355X (gfx950).
 *
 * Pages cited:
 *   [Lab06]    "LLM Lab notes 06: assembling a Megatron-style Transformer
 *              Block from scratch" (chat.ai-hpc.org), sections 1-5 and the
 *              listing's steps (1)-(8).
 *   [TP-block] "02 - How the whole Transformer block is sharded"
 *              (llm-infra-atlas.github.io), sections 1 MLP, 2 Attention,
 *              4 vocab-parallel cross entropy.
 *   [MLM-notes] "Megatron-LM" notes (huajishe.fun), ColumnParallelLinear /
 *              RowParallelLinear and the in-layer sharding figure.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership: the caller owns every buffer. All tensor pointers are DEVICE
 *   pointers (memory of the current HIP device) except the structs
 *   themselves, which are read on the host during the call. The library
 *   never allocates device memory; the sizes of the caller-provided `saved`
 *   and `scratch` buffers come from the *_bytes queries.
 * Layout: row-major, contiguous. Activations are [B, S, H] (token-major,
 *   T = B*S rows). Weights are [out, in]. Tensor pointers must be 16-byte
 *   aligned; the cross-entropy's per-token vectors (target, stats, loss,
 *   dloss) need only their element type's alignment.
 * Dtype: MTB_BF16 -- every tensor (activations, weights, biases, LN
 *   parameters, gradients, partial sums) is bf16, with fp32 accumulation
 *   inside; MTB_F32 -- everything fp32. LayerNorm statistics, the attention
 *   log-sum-exp and the cross-entropy statistics/loss are always fp32.
 * Streams: every kernel is enqueued on `hip_stream` (a hipStream_t; NULL =
 *   the default stream). Calls are asynchronous: no host synchronisation.
 *   Apart from the thread-local error message and the thread-local
 *   benchmark trace (mtb_trace_arm), the library holds no mutable global
 *   state, so calls on different streams with different buffers may run
 *   concurrently.
 * Errors: argument checks run before any launch; on failure nothing is
 *   launched and MTB_EINVAL (bad pointer, size or alignment) or
 *   MTB_EUNSUPPORTED (a valid shape the library has no kernel for) is
 *   returned. MTB_EHIP reports a failed launch, MTB_ECOMM a failed
 *   reduction hook (nothing further is launched after it).
 *   mtb_last_error() gives a message for the last non-OK status of the
 *   calling thread.
 */
#ifndef MTB_H
#define MTB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mtb_status;
#define MTB_OK 0
#define MTB_EINVAL 1
#define MTB_EUNSUPPORTED 2
#define MTB_EHIP 3
#define MTB_ECOMM 4

/* dtypes */
#define MTB_F32 0
#define MTB_BF16 1

/* MLP activation ([Lab06] step (6): GELU; [TP-block] sec. 1: SwiGLU) */
#define MTB_ACT_GELU 0
#define MTB_ACT_SWIGLU 1

/* LayerNorm placement. PRE ([Lab06] sec. 2 listing, (2) and (5)): each
 * sublayer reads LN(stream) and adds to the un-normalised stream. POST (the
 * order the same notes, (2)(5) and sec. 5, call post-LN: residual first,
 * then LayerNorm, as in the original Transformer): h = LN1(x + attn(x)),
 * out = LN2(h + mlp(h)). */
#define MTB_NORM_PRE 0
#define MTB_NORM_POST 1

/* Dropout ([TP-block] sec. 5). Inside the tensor-parallel region (the
 * attention probabilities of the local heads) every rank needs its own mask
 * stream: seed + MTB_TP_SEED_OFFSET + tp_rank. Outside it (the hidden state
 * after the attention block and after the MLP, replicated on every rank) all
 * ranks must draw the same mask: the seed itself. The mask is counter-based,
 * a pure function of (stream, site, element, rng_offset), so the backward
 * regenerates the forward's mask and a recomputation reproduces it:
 *   word = Philox4x32-10 (Salmon et al., SC 2011) with counter
 *          (i / 4 low 32 bits, i / 4 high 32 bits, site, rng_offset) and key
 *          (stream low 32 bits, stream high 32 bits), output word i % 4;
 *   dropped iff word < floor(p * 2^32) (p the float in mtb_cfg); a kept value
 *   is scaled by 1 / (1 - p).
 * Element index i: attention ((b * q_heads + h) * seq + query) * seq + key
 * over the LOCAL heads; hidden token * hidden + column. The hidden dropout
 * applies to sum(partials) + bias before the residual add. */
#define MTB_TP_SEED_OFFSET 2718
#define MTB_DROP_SITE_ATTN 0
#define MTB_DROP_SITE_HIDDEN_ATTN 1
#define MTB_DROP_SITE_HIDDEN_MLP 2

/* reduction ops of the communication hook */
#define MTB_OP_SUM 0
#define MTB_OP_MAX 1

/* Phases of one pass. A pass has two reduction points ([TP-block] sec. 2:
 * two all-reduces forward, two backward); SEG0..SEG2 are the pieces
 * between them, so that the shards of a layer can be run one after another
 * on one GPU with the caller summing the partials. MTB_PHASE_ALL runs the
 * whole pass and calls the hook (or nothing, when comm is NULL) at the
 * reduction points. */
#define MTB_PHASE_ALL 0
#define MTB_PHASE_SEG0 1
#define MTB_PHASE_SEG1 2
#define MTB_PHASE_SEG2 3

/* One rank's share of the layer. head/ffn counts are LOCAL sizes.
 *   batch, seq: B, S (T = B*S tokens);  hidden: H (replicated);
 *   q_heads, kv_heads: local query / key-value heads (q_heads % kv_heads == 0;
 *     q head i reads kv head i / (q_heads / kv_heads), [TP-block] sec. 2 GQA);
 *   head_dim: d;  ffn: local MLP width F;
 *   act: MTB_ACT_*;  causal: 0/1 (key s' > query s masked);
 *   dtype: MTB_F32 / MTB_BF16;  ln_eps: LayerNorm epsilon (e.g. 1e-5);
 *   norm: MTB_NORM_PRE / MTB_NORM_POST;
 *   attn_dropout, hidden_dropout: probabilities in [0, 1) (0: off);
 *   tp_rank: this rank's index in its tensor-parallel group (>= 0);
 *   rng_offset: counter word 3 of every mask (advance it per layer / step);
 *   seed: the 64-bit seed shared by the tensor-parallel group.
 * Supported shapes (else MTB_EUNSUPPORTED):
 *   MTB_BF16: head_dim in {64, 128}; seq, hidden, ffn and q_heads*head_dim
 *     multiples of 64 (tokens, hidden and ffn need not be multiples of the
 *     128-wide tiles); hidden <= 8192.
 *   MTB_F32: head_dim in {32, 64, 128}; hidden and ffn multiples of 8; any
 *     seq (a plain fp32 path, for correctness-size problems).
 *   SwiGLU: ffn % 16 == 0 (the gate/up interleave). */
typedef struct mtb_cfg {
  int32_t batch, seq, hidden;
  int32_t q_heads, kv_heads, head_dim;
  int32_t ffn;
  int32_t act;
  int32_t causal;
  int32_t dtype;
  float ln_eps;
  int32_t norm;
  float attn_dropout, hidden_dropout;
  int32_t tp_rank;
  uint32_t rng_offset;
  uint64_t seed;
} mtb_cfg;

/* Weights of one rank's share, all [out, in] row-major, dtype of the cfg.
 *   ln1_g, ln1_b [H]        input LayerNorm gain/shift (NULL = 1 / 0)
 *   w_qkv [Nqkv, H]         column-parallel QKV, Nqkv = (nq + 2*nkv)*d, rows
 *                           [Q heads | K heads | V heads], d rows per head
 *                           ([TP-block] sec. 2: out dim q_proj + 2*kv_proj)
 *   b_qkv [Nqkv]            (NULL = none)
 *   w_o [H, nq*d]           row-parallel output projection ([TP-block] sec. 2)
 *   b_o [H]                 added once, after the reduction (NULL = none)
 *   ln2_g, ln2_b [H]        second LayerNorm (NULL = 1 / 0)
 *   w_fc1 [F, H] (GELU) or [2F, H] (SwiGLU): SwiGLU gate and up rows are
 *                           interleaved in blocks of 16: rows 32j..32j+15 are
 *                           gate features 16j..16j+15 and rows 32j+16..32j+31
 *                           the up features 16j..16j+15, so that one rank
 *                           holds matching gate/up slices ([TP-block] sec. 1)
 *   b_fc1 [F] or [2F]       same interleave (NULL = none)
 *   w_fc2 [H, F]            row-parallel ([Lab06] step (6))
 *   b_fc2 [H]               added once, after the reduction (NULL = none)
 * ln*_g and ln*_b must both be given or both be NULL. */
typedef struct mtb_weights {
  const void *ln1_g, *ln1_b;
  const void *w_qkv, *b_qkv;
  const void *w_o, *b_o;
  const void *ln2_g, *ln2_b;
  const void *w_fc1, *b_fc1;
  const void *w_fc2, *b_fc2;
} mtb_weights;

/* Gradient outputs, same shapes/layouts as mtb_weights. Each non-NULL
 * pointer is WRITTEN (not accumulated); NULL = not requested. A gradient
 * may be requested only if the matching weight is present. */
typedef struct mtb_grads {
  void *ln1_g, *ln1_b;
  void *w_qkv, *b_qkv;
  void *w_o, *b_o;
  void *ln2_g, *ln2_b;
  void *w_fc1, *b_fc1;
  void *w_fc2, *b_fc2;
} mtb_grads;

/* Reduction hook: all-reduce `count` elements of `buf` (device memory,
 * dtype MTB_F32/MTB_BF16) in place with `op` over the tensor-parallel group,
 * enqueued on `hip_stream`. Returns MTB_OK or any non-zero value on failure.
 * A NULL mtb_comm (or NULL allreduce) is the identity: one rank / TP = 1. */
typedef mtb_status (*mtb_allreduce_fn)(void *buf, int64_t count, int32_t dtype, int32_t op,
                                       void *hip_stream, void *user);
typedef struct mtb_comm {
  mtb_allreduce_fn allreduce;
  void *user;
} mtb_comm;

/* Bytes of the `saved` buffer that carries activations from mtb_block_fwd to
 * mtb_block_bwd, and of the `scratch` buffer both use. Returns 0 if the cfg
 * is invalid or unsupported. */
size_t mtb_block_saved_bytes(const mtb_cfg *cfg);
size_t mtb_block_scratch_bytes(const mtb_cfg *cfg);

/* Forward of one rank's share ([Lab06] sec. 2 steps (2)-(7), pre-LN order;
 * [TP-block] sec. 1-2 column -> row sharding):
 *   a = LN1(x); qkv = a Wqkv^T + b_qkv; per head O = softmax(Q K^T/sqrt(d)) V
 *   (causal optional, GQA by head groups); p_attn = O Wo^T  [reduction g1];
 *   h = x + sum(p_attn) + b_o; c = LN2(h); m = GELU(c W1^T + b1) or
 *   silu(gate)*up; p_mlp = m W2^T  [reduction g2]; out = h + sum(p_mlp) + b2.
 * MTB_NORM_POST: qkv from x itself; h = LN1(x + sum(p_attn) + b_o) is the MLP
 *   input; out = LN2(h + sum(p_mlp) + b2). Same phases and reduction points.
 * Arguments:
 *   x [B,S,H]           block input (read in SEG0, SEG1; must be unchanged
 *                       between the phases of one pass)
 *   reduced_in [B,S,H]  SEG1: the sum over ranks of the SEG0 outputs;
 *                       SEG2: the sum over ranks of the SEG1 outputs;
 *                       ignored (may be NULL) for ALL and SEG0
 *   out [B,S,H]         ALL/SEG2: block output; SEG0: this rank's p_attn;
 *                       SEG1: this rank's p_mlp
 *   saved               mtb_block_saved_bytes(cfg) bytes, written here, read
 *                       by mtb_block_bwd; one per rank
 *   scratch             mtb_block_scratch_bytes(cfg) bytes; holds state
 *                       between the phases of one pass: one per rank
 *   comm                reduction hook used by MTB_PHASE_ALL (NULL = identity)
 * out may not alias x, reduced_in, saved or scratch. */
mtb_status mtb_block_fwd(const mtb_cfg *cfg, const mtb_weights *w, int32_t phase,
                         const void *x, const void *reduced_in, void *out,
                         void *saved, void *scratch, const mtb_comm *comm, void *hip_stream);

/* Backward of the same share for the cotangent dout = dL/d out [B,S,H].
 * Reductions follow the conjugate placement: a row-parallel output's sum is
 * the identity in the backward; a column-parallel input's gradient is
 * summed over ranks -- once for the fc1 input (dc) and once for the QKV input
 * (da) ([TP-block] sec. 2: two reductions backward).
 *   SEG0: fc2 and fc1 backward -> dx := this rank's dc partial
 *   SEG1: reduced_in = sum of dc; LN2 backward + residual, projection,
 *         attention and QKV backward -> dx := this rank's da partial
 *   SEG2: reduced_in = sum of da; LN1 backward + residual -> dx
 *   ALL:  the whole pass, hook at the two points -> dx
 * MTB_NORM_POST: SEG0 starts with LN2's backward; SEG1 runs LN1's backward
 *   of (residual + sum of dc) before the attention; SEG2 adds the sum of da
 *   to LN1's input gradient -> dx. LN2 gradients are written in SEG0, LN1's
 *   in SEG1.
 * x and saved are those of the matching mtb_block_fwd; dout must be
 * unchanged across the phases, and the same scratch passed to all of them.
 * Weight gradients are written in the phase that computes them (fc1/fc2 in
 * SEG0; LN2, projection, QKV in SEG1; LN1 in SEG2). dx may not alias any
 * input. */
mtb_status mtb_block_bwd(const mtb_cfg *cfg, const mtb_weights *w, int32_t phase,
                         const void *x, const void *saved, const void *dout,
                         const void *reduced_in, void *dx, const mtb_grads *grads,
                         void *scratch, const mtb_comm *comm, void *hip_stream);

/* Vocab-parallel cross-entropy ([TP-block] sec. 4) on one vocab shard.
 *   logits [n_tokens, v_local] (dtype), this shard's vocab ids
 *     [v_start, v_start + v_local); target [n_tokens] int64 GLOBAL ids in
 *     [0, V) (out-of-shard targets are normal input).
 * Phases:
 *   MTB_XENT_PARTIAL: one pass over the logits; stats[0..3n) :=
 *     (m_r, s_r, t_r) per token: local row max, sum_j exp(z - m_r), and the
 *     target logit z[target - v_start] if it lies in this shard, else 0.
 *   MTB_XENT_FINISH: stats holds the COMBINED (M, S, T) over all shards
 *     (see mtb_vocab_xent_combine, or the hook). Writes loss[n] =
 *     log S + M - T if loss != NULL, and, if dlogits != NULL,
 *     dlogits = (exp(z - M)/S - onehot(target)) * dloss[n]  (dloss != NULL).
 *   MTB_XENT_ALL: PARTIAL, then the hook's MAX of m, the local rescale
 *     s *= exp(m_r - M), the hook's SUMs of s and t, then FINISH.
 *     With a hook, stats must hold 4n floats (the last n keep this
 *     shard's max between the MAX and the rescale); with NULL comm 3n.
 *     (The [3][n] statistics layout is the same in every phase; the fourth
 *     row exists only because the hook reduces in place.)
 * dlogits may alias logits (read-before-write per element). */
#define MTB_XENT_PARTIAL 0
#define MTB_XENT_FINISH 1
#define MTB_XENT_ALL 2
mtb_status mtb_vocab_xent(int64_t n_tokens, int64_t v_local, int64_t v_start, int32_t dtype,
                          int32_t phase, const void *logits, const int64_t *target, float *stats,
                          float *loss, const float *dloss, void *dlogits, const mtb_comm *comm,
                          void *hip_stream);

/* The three reductions of [TP-block] sec. 4 over R shard statistics, as a
 * collective would give them: shard_stats [R][3][n] from MTB_XENT_PARTIAL
 * -> stats [3][n] = (M = max_r m_r, S = sum_r s_r exp(m_r - M),
 * T = sum_r t_r), and loss[n] = log S + M - T (if loss != NULL). */
mtb_status mtb_vocab_xent_combine(int64_t n_tokens, int32_t n_shards, const float *shard_stats,
                                  float *stats, float *loss, void *hip_stream);

/* Vocab-parallel output layer (LM head) fused with the vocab-parallel
 * cross-entropy ([TP-block] sec. 4 computes the loss from vocab-sharded
 * logits; here they come from this rank's vocab slice of the [V, hidden]
 * output embedding, rows [v_start, v_start + v_local), as z = h w^T, a
 * column-parallel linear). bf16 only; n_tokens, hidden, v_local multiples of
 * 8; h [n_tokens][hidden], w [v_local][hidden], 16-byte aligned.
 *
 * Forward: the logits are computed tile by tile and each tile is reduced in
 * the GEMM epilogue to per-token (max, sum exp, target logit); the
 * [n_tokens, v_local] logits are never stored. Then, exactly as
 * mtb_vocab_xent(MTB_XENT_ALL): stats [3][n_tokens] ([4][n_tokens] with a
 * hook) ends up holding the
 * combined (M, S, T) over the shards (the hook's MAX, local rescale, SUM,
 * SUM; NULL comm: one shard), and loss[n] = log S + M - T if loss != NULL.
 *
 * Backward, with the combined stats of the forward and dloss [n_tokens]:
 * recomputes the logits in a GEMM whose epilogue writes
 * dz = (exp(z - M)/S - onehot(target)) * dloss (bf16, in the workspace), then
 * dw = dz^T h [v_local][hidden] (if dw != NULL) and dh = dz w
 * [n_tokens][hidden] (if dh != NULL) -- this shard's partial of the input
 * gradient, summed over the shards by the hook (SUM, bf16). At least one of
 * dh, dw. Workspace: mtb_lmhead_xent_workspace_bytes (device, caller-owned,
 * 16-byte aligned; the same size serves both calls).
 *
 * logits (optional, bf16 [n_tokens][v_local]): trades memory for the
 * backward's recompute. Given to the forward, the logits are stored there
 * (rounded to bf16, and the statistics are those of the stored values, as
 * mtb_vocab_xent would see them); given to the backward (the same buffer),
 * no logits GEMM runs: dz is formed in place in `logits` (which it
 * overwrites) and the workspace may be NULL. NULL in both: the logits are
 * never stored. */
size_t mtb_lmhead_xent_workspace_bytes(int64_t n_tokens, int64_t hidden, int64_t v_local);
mtb_status mtb_lmhead_xent_fwd(int64_t n_tokens, int64_t hidden, int64_t v_local, int64_t v_start,
                               int32_t dtype, const void *h, const void *w, const int64_t *target,
                               float *stats, float *loss, void *logits, void *workspace,
                               const mtb_comm *comm, void *hip_stream);
mtb_status mtb_lmhead_xent_bwd(int64_t n_tokens, int64_t hidden, int64_t v_local, int64_t v_start,
                               int32_t dtype, const void *h, const void *w, const int64_t *target,
                               const float *stats, const float *dloss, void *logits, void *dh,
                               void *dw, void *workspace, const mtb_comm *comm, void *hip_stream);

/* Vocab-parallel input embedding ([TP-block] sec. 3) on one vocab shard:
 * this rank holds rows [v_start, v_start + v_local) of the [vocab, hidden]
 * table.
 *   ids [n_tokens] int64 GLOBAL token ids (any value: ids outside this
 *     shard's range, negative or beyond the vocab, select nothing here);
 *   table [v_local][hidden] (dtype), out [n_tokens][hidden] (dtype).
 * Forward: out[t] = table[ids[t] - v_start] when the id lies in the shard,
 * else a zero row; then, with a hook, out is all-reduced (SUM) over the
 * shards -- the masks make exactly one shard contribute each token's row.
 * NULL comm: identity (one shard). hidden % 8 == 0; table, out 16-byte and
 * ids 8-byte aligned; n_tokens, v_local < 2^31. */
mtb_status mtb_vocab_embed_fwd(int64_t n_tokens, int64_t v_local, int64_t v_start, int64_t hidden,
                               int32_t dtype, const int64_t *ids, const void *table, void *out,
                               const mtb_comm *comm, void *hip_stream);

/* Device workspace (bytes, caller-owned) that mtb_vocab_embed_bwd needs:
 * 8 bytes per table row of the shard (a token count and a first token);
 * 0 when n_tokens or v_local is outside 1 .. 2^31 - 1. */
size_t mtb_vocab_embed_bwd_workspace_bytes(int64_t n_tokens, int64_t v_local);

/* Backward of the embedding: the all-reduce's backward is the identity, so
 * dout [n_tokens][hidden] is the full (replicated) gradient of out. Writes
 * dtable[v] = sum of dout[t] over the tokens t with ids[t] == v_start + v,
 * accumulated in fp32 in increasing t (deterministic), rounded once; rows no
 * token selects are written as zeros. Same layout and alignment rules as the
 * forward; workspace 16-byte aligned. */
mtb_status mtb_vocab_embed_bwd(int64_t n_tokens, int64_t v_local, int64_t v_start, int64_t hidden,
                               int32_t dtype, const int64_t *ids, const void *dout, void *dtable,
                               void *workspace, void *hip_stream);

/* The same backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; the per-row (count, first token) pairs
 * live in a device array of the library, one per GPU, allocated with the
 * library's code and held until the process ends (8 bytes per row,
 * MTB_EMBED_NOALLOC_MAX_ROWS rows = 2 MiB). The call allocates nothing; the
 * first call on a device looks the array's address up (hipGetSymbolAddress)
 * with that device current. v_local above MTB_EMBED_NOALLOC_MAX_ROWS returns
 * MTB_EUNSUPPORTED and launches nothing. Every call on one GPU uses the same
 * array (the kernels reinitialise it each call): calls that may overlap on
 * one GPU -- different streams, or different host threads -- race and give
 * wrong results; serialise them. Output and arguments otherwise exactly as
 * mtb_vocab_embed_bwd. */
#define MTB_EMBED_NOALLOC_MAX_ROWS 262144
mtb_status mtb_vocab_embed_bwd_noalloc(int64_t n_tokens, int64_t v_local, int64_t v_start,
                                       int64_t hidden, int32_t dtype, const int64_t *ids,
                                       const void *dout, void *dtable, void *hip_stream);

/* Benchmark instrumentation. The armed state is per host thread (like the
 * error message): only calls made on the arming thread are traced, and
 * other threads' calls are unaffected. While armed, every launch of the kernel class `what` records
 * begin_events[i] before it and end_events[i] after it on the launch's
 * stream, for i = 0, 1, ... up to n - 1 (later launches are not recorded).
 * The events are caller-created hipEvent_t handles. mtb_trace_disarm()
 * stops recording and returns how many pairs were recorded. */
#define MTB_TRACE_NONE 0
#define MTB_TRACE_FC1_FWD 1   /* column-parallel fc1 GEMM + activation, forward */
#define MTB_TRACE_ATTN_FWD 2  /* attention forward */
#define MTB_TRACE_LN1_FWD 3   /* input LayerNorm forward */
#define MTB_TRACE_FC2_WGRAD 4 /* fc2 weight-gradient GEMM (with fc1's when the two run as one launch) */
/* Segments of MTB_PHASE_ALL calls (the attention / FFN / backward breakdown
 * of [Lab06] sec. 4): */
#define MTB_TRACE_ATTN_SEG 5  /* forward LN1 .. projection (with the fused residual) */
#define MTB_TRACE_FFN_SEG 6   /* forward LN2 .. fc2 (with the residual) */
#define MTB_TRACE_BWD 7       /* the whole backward call */
#define MTB_TRACE_LN1_BWD 8   /* input LayerNorm backward + residual-gradient add */
mtb_status mtb_trace_arm(int32_t what, void *const *begin_events, void *const *end_events, int32_t n);
int32_t mtb_trace_disarm(void);

/* Message for the last non-OK status returned on the calling thread. */
const char *mtb_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MTB_H */
