// libmtb C ABI: argument validation, the layout of the caller-provided
// `saved` / `scratch` buffers, and the order of kernel launches for the
// forward and backward pass of one tensor-parallel rank's share of the block.
//
// Block structure: [Lab06] sec. 2 listing steps (2)-(8) in its pre-LN order,
// or the post-LN order its notes (2)(5) describe (residual first, then LN);
// sharding and the reduction points: [TP-block] sec. 1-2 (column-parallel
// QKV and fc1, row-parallel projection and fc2, two all-reduces forward and
// two backward); vocab-parallel cross-entropy: [TP-block] sec. 4.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "kernels.h"
#include "mtb.h"

using namespace mtb;

namespace {

thread_local std::string g_err;

mtb_status fail(mtb_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

#define MTB_HIP(call)                                                                       \
  do {                                                                                      \
    hipError_t e_ = (call);                                                                 \
    if (e_ != hipSuccess)                                                                   \
      return fail(MTB_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));                 \
  } while (0)

struct Dims {
  int64_t B, S, H, nq, nkv, d, F, Fu, Nqkv, T, NO;
  int64_t es;  // element size
  int dt;      // MTB_F32 / MTB_BF16
  int act, causal;
  float eps;
  bool post;   // post-LN order
  // dropout ([TP-block] sec. 5): attention probabilities (this rank's
  // stream), hidden state after the attention and after the MLP (the stream
  // every rank shares)
  Drop dattn, dh1, dh2;
};

Drop make_drop(float p, uint64_t key, uint32_t site, uint32_t offset) {
  Drop d;
  if (p > 0.f) {
    const double t = floor((double)p * 4294967296.0);
    d.thr = t >= 4294967295.0 ? 0xffffffffu : (uint32_t)t;
    d.scale = (float)(1.0 / (1.0 - (double)p));
  }
  d.k0 = (uint32_t)key;
  d.k1 = (uint32_t)(key >> 32);
  d.site = site;
  d.offset = offset;
  return d;
}

mtb_status check_cfg(const mtb_cfg* c, Dims& d) {
  if (!c) return fail(MTB_EINVAL, "cfg is NULL");
  if (c->batch <= 0 || c->seq <= 0 || c->hidden <= 0 || c->q_heads <= 0 || c->kv_heads <= 0 ||
      c->head_dim <= 0 || c->ffn <= 0)
    return fail(MTB_EINVAL, "cfg sizes must be positive");
  if (c->q_heads % c->kv_heads)
    return fail(MTB_EINVAL, "q_heads (%d) must be a multiple of kv_heads (%d)", c->q_heads,
                c->kv_heads);
  if (c->act != MTB_ACT_GELU && c->act != MTB_ACT_SWIGLU)
    return fail(MTB_EINVAL, "act must be MTB_ACT_GELU or MTB_ACT_SWIGLU");
  if (c->causal != 0 && c->causal != 1) return fail(MTB_EINVAL, "causal must be 0 or 1");
  if (c->dtype != MTB_F32 && c->dtype != MTB_BF16) return fail(MTB_EINVAL, "bad dtype %d", c->dtype);
  if (!(c->ln_eps > 0.f) || c->ln_eps > 1.f) return fail(MTB_EINVAL, "ln_eps must be in (0, 1]");
  if (c->norm != MTB_NORM_PRE && c->norm != MTB_NORM_POST)
    return fail(MTB_EINVAL, "norm must be MTB_NORM_PRE or MTB_NORM_POST");
  if (!(c->attn_dropout >= 0.f && c->attn_dropout < 1.f) ||
      !(c->hidden_dropout >= 0.f && c->hidden_dropout < 1.f))
    return fail(MTB_EINVAL, "dropout probabilities must be in [0, 1)");
  if (c->tp_rank < 0) return fail(MTB_EINVAL, "tp_rank must be >= 0");
  d.B = c->batch; d.S = c->seq; d.H = c->hidden; d.nq = c->q_heads; d.nkv = c->kv_heads;
  d.d = c->head_dim; d.F = c->ffn; d.act = c->act; d.causal = c->causal; d.dt = c->dtype;
  d.eps = c->ln_eps;
  d.post = c->norm == MTB_NORM_POST;
  d.dattn = make_drop(c->attn_dropout, c->seed + MTB_TP_SEED_OFFSET + (uint64_t)c->tp_rank,
                      MTB_DROP_SITE_ATTN, c->rng_offset);
  d.dh1 = make_drop(c->hidden_dropout, c->seed, MTB_DROP_SITE_HIDDEN_ATTN, c->rng_offset);
  d.dh2 = make_drop(c->hidden_dropout, c->seed, MTB_DROP_SITE_HIDDEN_MLP, c->rng_offset);
  d.Fu = d.act == MTB_ACT_SWIGLU ? 2 * d.F : d.F;
  d.Nqkv = (d.nq + 2 * d.nkv) * d.d;
  d.T = d.B * d.S;
  d.NO = d.nq * d.d;
  d.es = d.dt == MTB_BF16 ? 2 : 4;
  if (d.T > (1 << 30) || d.H > 8192 || d.Nqkv > (1 << 20) || d.Fu > (1 << 24))
    return fail(MTB_EUNSUPPORTED, "sizes beyond the library's limits (T <= 2^30, hidden <= 8192)");
  if (d.act == MTB_ACT_SWIGLU && d.F % 16)
    return fail(MTB_EUNSUPPORTED, "SwiGLU needs ffn %% 16 == 0 (gate/up interleave of 16)");
  if (d.dt == MTB_BF16) {
    if (d.d != 64 && d.d != 128)
      return fail(MTB_EUNSUPPORTED, "bf16 path supports head_dim 64 or 128, got %d", c->head_dim);
    if (d.S % 64 || d.H % 64 || d.F % 64 || d.NO % 64)
      return fail(MTB_EUNSUPPORTED,
                  "bf16 path needs seq, hidden, ffn and q_heads*head_dim multiples of 64");
  } else {
    if (d.d != 32 && d.d != 64 && d.d != 128)
      return fail(MTB_EUNSUPPORTED, "fp32 path supports head_dim 32, 64 or 128, got %d",
                  c->head_dim);
    if (d.H % 8 || d.F % 8) return fail(MTB_EUNSUPPORTED, "fp32 path needs hidden, ffn %% 8 == 0");
  }
  return MTB_OK;
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

// Saved activations. Pre-LN: a = LN1(x), h = x + attn, c = LN2(h).
// Post-LN: h = r1 = x + attn, c = LN1(r1) (the MLP input), a = r2 = c + mlp
// (the second LayerNorm's input); mu/rstd 1 and 2 belong to LN1 and LN2.
struct Saved {
  size_t a, mu1, rs1, qkv, O, lse, h, mu2, rs2, c, u, m, total;
};
Saved saved_layout(const Dims& d) {
  Saved s;
  size_t o = 0;
  const size_t e = d.es, T = d.T;
  s.a = o; o += al(T * d.H * e);
  s.mu1 = o; o += al(T * 4);
  s.rs1 = o; o += al(T * 4);
  s.qkv = o; o += al(T * d.Nqkv * e);
  s.O = o; o += al(T * d.NO * e);
  s.lse = o; o += al((size_t)d.B * d.nq * d.S * 4);
  s.h = o; o += al(T * d.H * e);
  s.mu2 = o; o += al(T * 4);
  s.rs2 = o; o += al(T * 4);
  s.c = o; o += al(T * d.H * e);
  s.u = o; o += al(T * d.Fu * e);
  s.m = o; o += al(T * d.F * e);
  s.total = o;
  return s;
}

// Weight gradients as gemm_wgrad_pair products (operands may be null when only
// sizes are needed), contractions over the tokens: dWqkv [Nqkv][H] = dqkv^T a,
// dWo [H][nq d] = dA^T O, dW2 [H][F] = G^T m, dW1 [Fu][H] = du^T c.
GemmProb wgrad_qkv(const Dims& d, const void* dqkv, const void* a) {
  GemmProb p{(int)d.Nqkv, (int)d.H, (int)d.T, dqkv, (int)d.Nqkv, a, (int)d.H, Epi()};
  p.e.ldo = (int)d.H;
  return p;
}
GemmProb wgrad_proj(const Dims& d, const void* dA, const void* O) {
  GemmProb p{(int)d.H, (int)d.NO, (int)d.T, dA, (int)d.H, O, (int)d.NO, Epi()};
  p.e.ldo = (int)d.NO;
  return p;
}
GemmProb wgrad_fc2(const Dims& d, const void* G, const void* m) {
  GemmProb p{(int)d.H, (int)d.F, (int)d.T, G, (int)d.H, m, (int)d.F, Epi()};
  p.e.ldo = (int)d.F;
  return p;
}
GemmProb wgrad_fc1(const Dims& d, const void* du, const void* c) {
  GemmProb p{(int)d.Fu, (int)d.H, (int)d.T, du, (int)d.Fu, c, (int)d.H, Epi()};
  p.e.ldo = (int)d.H;
  return p;
}

struct Scratch {
  size_t dh, dr, gm, p, du, dm, dO, Dbuf, dqkv, part, red, ws, total;
};
Scratch scratch_layout(const Dims& d) {
  Scratch s;
  size_t o = 0;
  const size_t e = d.es, T = d.T;
  s.dh = o; o += al(T * d.H * e);       // pre: dh, SEG1 -> SEG2; post: dr2, SEG0 -> SEG1
  s.dr = o; o += d.post ? al(T * d.H * e) : 0;   // post: dr1, SEG1 -> SEG2
  s.gm = o; o += d.dh1.thr ? al(T * d.H * e) : 0;  // hidden dropout: masked upstream gradient
  s.p = o; o += al(T * d.H * e);        // partial sums (p_attn, p_mlp, dc, da)
  s.du = o; o += al(T * d.Fu * e);
  s.dm = o; o += d.dt == MTB_F32 ? al(T * d.F * e) : 0;
  s.dO = o; o += al(T * d.NO * e);
  s.Dbuf = o; o += al((size_t)d.B * d.nq * d.S * 4);
  s.dqkv = o; o += al(T * d.Nqkv * e);
  s.part = o; o += (d.dt == MTB_BF16 && d.nq != d.nkv) ? al((size_t)d.B * d.nq * d.S * 2 * d.d * 4) : 0;
  int64_t nmax = d.H > d.Fu ? d.H : d.Fu;
  if (d.Nqkv > nmax) nmax = d.Nqkv;
  s.red = o; o += al((size_t)colsum_splits((int)d.T) * nmax * 4);
  // split-contraction partial tiles (one GEMM, or one grouped pair, at a
  // time): the largest any of them asks for
  const int dt = d.dt, T32 = (int)d.T, H = (int)d.H, Nq = (int)d.Nqkv, NO = (int)d.NO,
            F = (int)d.F, Fu = (int)d.Fu;
  const int act_f = d.act == MTB_ACT_GELU ? EPI_GELU : EPI_SWIGLU;
  const int act_b = d.act == MTB_ACT_GELU ? EPI_DGELU : EPI_DSWIGLU;
  const size_t need[] = {
      gemm_ws_bytes(dt, T32, Nq, H, true, true, EPI_STORE),    // QKV
      gemm_ws_bytes(dt, T32, H, NO, true, true, EPI_STORE),    // projection
      gemm_ws_bytes(dt, T32, Fu, H, true, true, act_f),        // fc1
      gemm_ws_bytes(dt, T32, H, F, true, true, EPI_STORE),     // fc2
      gemm_ws_bytes(dt, T32, F, H, true, false, act_b),        // fc2 dgrad
      gemm_ws_bytes(dt, T32, H, Fu, true, false, EPI_STORE),   // fc1 dgrad
      gemm_ws_bytes(dt, T32, NO, H, true, false, EPI_STORE),   // projection dgrad
      gemm_ws_bytes(dt, T32, H, Nq, true, false, EPI_STORE),   // QKV dgrad
      gemm_ws_bytes(dt, H, F, T32, false, false, EPI_STORE),   // weight gradients
      gemm_ws_bytes(dt, Fu, H, T32, false, false, EPI_STORE),
      gemm_ws_bytes(dt, H, NO, T32, false, false, EPI_STORE),
      gemm_ws_bytes(dt, Nq, H, T32, false, false, EPI_STORE),
      gemm_wgrad_pair_ws_bytes(dt, wgrad_qkv(d, nullptr, nullptr), wgrad_proj(d, nullptr, nullptr)),
      gemm_wgrad_pair_ws_bytes(dt, wgrad_fc2(d, nullptr, nullptr), wgrad_fc1(d, nullptr, nullptr))};
  size_t ws = 0;
  for (size_t v : need) ws = v > ws ? v : ws;
  s.ws = o; o += al(ws);
  s.total = o;
  return s;
}

bool misaligned(const void* p, uintptr_t a = 16) { return ((uintptr_t)p & (a - 1)) != 0; }

#define MTB_REQ(p, name)                                                             \
  do {                                                                               \
    if (!(p)) return fail(MTB_EINVAL, "%s is NULL", name);                           \
    if (misaligned(p)) return fail(MTB_EINVAL, "%s is not 16-byte aligned", name);   \
  } while (0)
#define MTB_OPT(p, name)                                                             \
  do {                                                                               \
    if ((p) && misaligned(p)) return fail(MTB_EINVAL, "%s is not 16-byte aligned", name); \
  } while (0)
// small per-token vectors: natural alignment of their element type
#define MTB_REQ_A(p, name, a)                                                        \
  do {                                                                               \
    if (!(p)) return fail(MTB_EINVAL, "%s is NULL", name);                           \
    if (misaligned(p, a)) return fail(MTB_EINVAL, "%s is not %d-byte aligned", name, (int)(a)); \
  } while (0)
#define MTB_OPT_A(p, name, a)                                                        \
  do {                                                                               \
    if ((p) && misaligned(p, a)) return fail(MTB_EINVAL, "%s is not %d-byte aligned", name, (int)(a)); \
  } while (0)

mtb_status check_weights(const mtb_weights* w) {
  if (!w) return fail(MTB_EINVAL, "weights is NULL");
  MTB_REQ(w->w_qkv, "w_qkv");
  MTB_REQ(w->w_o, "w_o");
  MTB_REQ(w->w_fc1, "w_fc1");
  MTB_REQ(w->w_fc2, "w_fc2");
  MTB_OPT(w->b_qkv, "b_qkv"); MTB_OPT(w->b_o, "b_o"); MTB_OPT(w->b_fc1, "b_fc1");
  MTB_OPT(w->b_fc2, "b_fc2"); MTB_OPT(w->ln1_g, "ln1_g"); MTB_OPT(w->ln1_b, "ln1_b");
  MTB_OPT(w->ln2_g, "ln2_g"); MTB_OPT(w->ln2_b, "ln2_b");
  if ((!w->ln1_g) != (!w->ln1_b) || (!w->ln2_g) != (!w->ln2_b))
    return fail(MTB_EINVAL, "LayerNorm gain and shift must be given together");
  return MTB_OK;
}

mtb_status call_hook(const mtb_comm* comm, void* buf, int64_t count, int dt, int op, hipStream_t st) {
  if (!comm || !comm->allreduce) return MTB_OK;
  const mtb_status s = comm->allreduce(buf, count, dt, op, (void*)st, comm->user);
  if (s != MTB_OK) return fail(MTB_ECOMM, "reduction hook returned %d", (int)s);
  return MTB_OK;
}

char* P(void* base, size_t off) { return (char*)base + off; }

// benchmark trace (see mtb_trace_arm)
struct Trace {
  int what = MTB_TRACE_NONE;
  void* const* b = nullptr;
  void* const* e = nullptr;
  int n = 0, i = 0;
};
thread_local Trace g_trace;  // per host thread, like the error message

void trace_begin(int what, hipStream_t st) {
  if (g_trace.what == what && g_trace.i < g_trace.n) hipEventRecord((hipEvent_t)g_trace.b[g_trace.i], st);
}
void trace_end(int what, hipStream_t st) {
  if (g_trace.what == what && g_trace.i < g_trace.n) hipEventRecord((hipEvent_t)g_trace.e[g_trace.i++], st);
}

}  // namespace

namespace {
mtb_status check_embed(int64_t n, int64_t v, int64_t v0, int64_t h, int32_t dtype) {
  if (n <= 0 || v <= 0 || v0 < 0 || h <= 0)
    return fail(MTB_EINVAL, "n_tokens, v_local, hidden must be > 0 and v_start >= 0");
  if (dtype != MTB_F32 && dtype != MTB_BF16) return fail(MTB_EINVAL, "bad dtype %d", dtype);
  if (h % 8 != 0) return fail(MTB_EUNSUPPORTED, "hidden %lld is not a multiple of 8", (long long)h);
  if (n > 0x7fffffff || v > 0x7fffffff || h > 0x7fffffff)
    return fail(MTB_EUNSUPPORTED, "n_tokens, v_local and hidden must be below 2^31");
  return MTB_OK;
}
mtb_status check_lmhead(int64_t n, int64_t h, int64_t v, int64_t v0, int32_t dtype) {
  if (n <= 0 || h <= 0 || v <= 0 || v0 < 0)
    return fail(MTB_EINVAL, "n_tokens, hidden, v_local must be > 0 and v_start >= 0");
  if (dtype != MTB_BF16)
    return fail(dtype == MTB_F32 ? MTB_EUNSUPPORTED : MTB_EINVAL, "the LM head runs in bf16 only");
  if (n % 8 || h % 8 || v % 8)
    return fail(MTB_EUNSUPPORTED, "n_tokens, hidden and v_local must be multiples of 8");
  if (n > 0x7fffffff || h > 0x7fffffff || v > 0x7fffffff)
    return fail(MTB_EUNSUPPORTED, "n_tokens, hidden and v_local must be below 2^31");
  return MTB_OK;
}

int lmhead_tiles(int64_t n, int64_t h, int64_t v) {
  const int bn = gemm_tile_n((int)n, (int)v, (int)h, true, true, EPI_XENT_STATS);
  return (int)((v + bn - 1) / bn);
}

}  // namespace

extern "C" {

const char* mtb_last_error(void) { return g_err.c_str(); }

mtb_status mtb_trace_arm(int32_t what, void* const* begin_events, void* const* end_events, int32_t n) {
  if (what < MTB_TRACE_NONE || what > MTB_TRACE_LN1_BWD || n < 0)
    return fail(MTB_EINVAL, "bad trace request");
  if (n > 0 && (!begin_events || !end_events)) return fail(MTB_EINVAL, "trace events are NULL");
  g_trace.what = what;
  g_trace.b = begin_events;
  g_trace.e = end_events;
  g_trace.n = n;
  g_trace.i = 0;
  return MTB_OK;
}

int32_t mtb_trace_disarm(void) {
  const int32_t k = g_trace.i;
  g_trace = Trace();
  return k;
}

size_t mtb_block_saved_bytes(const mtb_cfg* cfg) {
  Dims d;
  if (check_cfg(cfg, d) != MTB_OK) return 0;
  return saved_layout(d).total;
}

size_t mtb_block_scratch_bytes(const mtb_cfg* cfg) {
  Dims d;
  if (check_cfg(cfg, d) != MTB_OK) return 0;
  return scratch_layout(d).total;
}

mtb_status mtb_block_fwd(const mtb_cfg* cfg, const mtb_weights* w, int32_t phase, const void* x,
                         const void* reduced_in, void* out, void* saved, void* scratch,
                         const mtb_comm* comm, void* hip_stream) {
  Dims d;
  mtb_status s = check_cfg(cfg, d);
  if (s != MTB_OK) return s;
  if (phase < MTB_PHASE_ALL || phase > MTB_PHASE_SEG2) return fail(MTB_EINVAL, "bad phase %d", phase);
  if ((s = check_weights(w)) != MTB_OK) return s;
  MTB_REQ(x, "x");
  MTB_REQ(out, "out");
  MTB_REQ(saved, "saved");
  MTB_REQ(scratch, "scratch");
  if (phase == MTB_PHASE_SEG1 || phase == MTB_PHASE_SEG2) MTB_REQ(reduced_in, "reduced_in");
  if (out == x || out == reduced_in || out == saved || out == scratch)
    return fail(MTB_EINVAL, "out may not alias an input or a work buffer");

  hipStream_t st = (hipStream_t)hip_stream;
  const Saved L = saved_layout(d);
  const Scratch Z = scratch_layout(d);
  const int dt = d.dt;
  const int T = (int)d.T, H = (int)d.H, Nq = (int)d.Nqkv, NO = (int)d.NO, F = (int)d.F,
            Fu = (int)d.Fu, S = (int)d.S;
  const bool bf = dt == MTB_BF16;
  const bool fused = phase == MTB_PHASE_ALL && !(comm && comm->allreduce);
  void* a = P(saved, L.a); float* mu1 = (float*)P(saved, L.mu1); float* rs1 = (float*)P(saved, L.rs1);
  void* qkv = P(saved, L.qkv);
  void* O = P(saved, L.O); float* lse = (float*)P(saved, L.lse);
  void* h = P(saved, L.h); float* mu2 = (float*)P(saved, L.mu2); float* rs2 = (float*)P(saved, L.rs2);
  void* c = P(saved, L.c); void* u = P(saved, L.u); void* m = P(saved, L.m);
  void* p = P(scratch, Z.p);
  void* ws = Z.total > Z.ws ? P(scratch, Z.ws) : nullptr;

  const bool all = phase == MTB_PHASE_ALL;
  const bool post = d.post;
  // the LayerNorm after the attention residual: LN2 (pre-LN) or LN1 (post-LN)
  const void* lnA_g = post ? w->ln1_g : w->ln2_g;
  const void* lnA_b = post ? w->ln1_b : w->ln2_b;
  float* muA = post ? mu1 : mu2;
  float* rsA = post ? rs1 : rs2;
  void* r2 = a;  // post-LN: the second LayerNorm's input
  if (phase == MTB_PHASE_ALL || phase == MTB_PHASE_SEG0) {
    if (all) trace_begin(MTB_TRACE_ATTN_SEG, st);
    if (!post) {
      // (2) input LayerNorm
      trace_begin(MTB_TRACE_LN1_FWD, st);
      MTB_HIP(ln_fwd(dt, T, H, x, nullptr, nullptr, w->ln1_g, w->ln1_b, nullptr, a, mu1, rs1, d.eps, st));
      trace_end(MTB_TRACE_LN1_FWD, st);
    }
    // column-parallel QKV on LN1(x) (pre-LN) or x (post-LN)
    Epi e;
    e.out = qkv; e.ldo = Nq; e.bias = w->b_qkv; e.ws = ws;
    MTB_HIP(gemm(dt, T, Nq, H, post ? x : a, H, true, w->w_qkv, H, true, e, st));
    // per-head attention over the local heads
    trace_begin(MTB_TRACE_ATTN_FWD, st);
    MTB_HIP(attn_fwd(dt, (int)d.B, S, (int)d.nq, (int)d.nkv, (int)d.d, d.causal, qkv, O, lse, st,
                     d.dattn));
    trace_end(MTB_TRACE_ATTN_FWD, st);
    // row-parallel projection: a partial sum, reduced at g1
    Epi ep;
    ep.ws = ws;
    if (fused) {  // identity reduction: fuse (4) residual, the bias and the dropout
      ep.out = h; ep.ldo = H; ep.bias = w->b_o; ep.resid = x; ep.ldr = H; ep.drop = d.dh1;
    } else {
      ep.out = phase == MTB_PHASE_SEG0 ? out : p; ep.ldo = H;
    }
    MTB_HIP(gemm(dt, T, H, NO, O, NO, true, w->w_o, NO, true, ep, st));
    if (phase == MTB_PHASE_SEG0) return MTB_OK;
    if (fused) {
      trace_end(MTB_TRACE_ATTN_SEG, st);
      trace_begin(MTB_TRACE_FFN_SEG, st);
      MTB_HIP(ln_fwd(dt, T, H, h, nullptr, nullptr, lnA_g, lnA_b, nullptr, c, muA, rsA, d.eps, st));
    } else {
      if ((s = call_hook(comm, p, d.T * d.H, dt, MTB_OP_SUM, st)) != MTB_OK) return s;
      trace_end(MTB_TRACE_ATTN_SEG, st);
      trace_begin(MTB_TRACE_FFN_SEG, st);
      MTB_HIP(ln_fwd(dt, T, H, x, p, w->b_o, lnA_g, lnA_b, h, c, muA, rsA, d.eps, st, d.dh1));
    }
  } else if (phase == MTB_PHASE_SEG1) {
    // g1 done by the caller: h = x + dropout(sum(p_attn) + b_o), then (5) LN2
    // (pre-LN) or LN1 (post-LN) of it
    MTB_HIP(ln_fwd(dt, T, H, x, reduced_in, w->b_o, lnA_g, lnA_b, h, c, muA, rsA, d.eps, st, d.dh1));
  }

  if (phase == MTB_PHASE_ALL || phase == MTB_PHASE_SEG1) {
    // column-parallel fc1 + activation
    if (bf) {
      Epi e;
      e.kind = d.act == MTB_ACT_GELU ? EPI_GELU : EPI_SWIGLU;
      e.out = u; e.ldo = Fu; e.out2 = m; e.ldo2 = F; e.bias = w->b_fc1; e.ws = ws;
      trace_begin(MTB_TRACE_FC1_FWD, st);
      MTB_HIP(gemm(dt, T, Fu, H, c, H, true, w->w_fc1, H, true, e, st));
      trace_end(MTB_TRACE_FC1_FWD, st);
    } else {
      Epi e;
      e.out = u; e.ldo = Fu; e.bias = w->b_fc1;
      MTB_HIP(gemm(dt, T, Fu, H, c, H, true, w->w_fc1, H, true, e, st));
      MTB_HIP(act_fwd(dt, d.act, T, F, u, m, st));
    }
    // (6) row-parallel fc2: a partial sum, reduced at g2; (7) residual onto
    // h (pre-LN) or onto the MLP input (post-LN, then LN2)
    Epi e;
    e.ws = ws;
    if (fused) {
      e.out = post ? r2 : out; e.ldo = H; e.bias = w->b_fc2; e.resid = post ? c : h; e.ldr = H;
      e.drop = d.dh2;
    } else {
      e.out = phase == MTB_PHASE_SEG1 ? out : p; e.ldo = H;
    }
    MTB_HIP(gemm(dt, T, H, F, m, F, true, w->w_fc2, F, true, e, st));
    if (fused) {
      if (post)
        MTB_HIP(ln_fwd(dt, T, H, r2, nullptr, nullptr, w->ln2_g, w->ln2_b, nullptr, out, mu2, rs2,
                       d.eps, st));
      trace_end(MTB_TRACE_FFN_SEG, st);
    }
    if (fused || phase == MTB_PHASE_SEG1) return MTB_OK;
    if ((s = call_hook(comm, p, d.T * d.H, dt, MTB_OP_SUM, st)) != MTB_OK) return s;
    if (post)
      MTB_HIP(ln_fwd(dt, T, H, c, p, w->b_fc2, w->ln2_g, w->ln2_b, r2, out, mu2, rs2, d.eps, st,
                     d.dh2));
    else
      MTB_HIP(add3(dt, T, H, h, p, w->b_fc2, out, st, d.dh2));
    trace_end(MTB_TRACE_FFN_SEG, st);
    return MTB_OK;
  }
  // SEG2: out = h + sum(p_mlp) + b2 (pre-LN), or LN2(c + sum(p_mlp) + b2)
  if (post)
    MTB_HIP(ln_fwd(dt, T, H, c, reduced_in, w->b_fc2, w->ln2_g, w->ln2_b, r2, out, mu2, rs2, d.eps,
                   st, d.dh2));
  else
    MTB_HIP(add3(dt, T, H, h, reduced_in, w->b_fc2, out, st, d.dh2));
  return MTB_OK;
}

mtb_status mtb_block_bwd(const mtb_cfg* cfg, const mtb_weights* w, int32_t phase, const void* x,
                         const void* saved, const void* dout, const void* reduced_in, void* dx,
                         const mtb_grads* grads, void* scratch, const mtb_comm* comm,
                         void* hip_stream) {
  Dims d;
  mtb_status s = check_cfg(cfg, d);
  if (s != MTB_OK) return s;
  if (phase < MTB_PHASE_ALL || phase > MTB_PHASE_SEG2) return fail(MTB_EINVAL, "bad phase %d", phase);
  if ((s = check_weights(w)) != MTB_OK) return s;
  MTB_REQ(x, "x");
  MTB_REQ(saved, "saved");
  MTB_REQ(dout, "dout");
  MTB_REQ(dx, "dx");
  MTB_REQ(scratch, "scratch");
  if (phase == MTB_PHASE_SEG1 || phase == MTB_PHASE_SEG2) MTB_REQ(reduced_in, "reduced_in");
  if (dx == x || dx == dout || dx == reduced_in || dx == saved || dx == scratch)
    return fail(MTB_EINVAL, "dx may not alias an input or a work buffer");
  mtb_grads g0 = {};
  const mtb_grads& g = grads ? *grads : g0;
  {
    const void* gp[12] = {g.ln1_g, g.ln1_b, g.w_qkv, g.b_qkv, g.w_o, g.b_o,
                          g.ln2_g, g.ln2_b, g.w_fc1, g.b_fc1, g.w_fc2, g.b_fc2};
    const void* wp[12] = {w->ln1_g, w->ln1_b, w->w_qkv, w->b_qkv, w->w_o, w->b_o,
                          w->ln2_g, w->ln2_b, w->w_fc1, w->b_fc1, w->w_fc2, w->b_fc2};
    for (int i = 0; i < 12; ++i) {
      if (gp[i] && misaligned(gp[i])) return fail(MTB_EINVAL, "gradient %d is not 16-byte aligned", i);
      if (gp[i] && !wp[i]) return fail(MTB_EINVAL, "gradient %d requested for an absent weight", i);
    }
  }

  hipStream_t st = (hipStream_t)hip_stream;
  const Saved L = saved_layout(d);
  const Scratch Z = scratch_layout(d);
  const int dt = d.dt;
  const int T = (int)d.T, H = (int)d.H, Nq = (int)d.Nqkv, NO = (int)d.NO, F = (int)d.F,
            Fu = (int)d.Fu, S = (int)d.S;
  const bool bf = dt == MTB_BF16;
  char* sv = (char*)saved;
  const void* a = sv + L.a; const float* mu1 = (const float*)(sv + L.mu1);
  const float* rs1 = (const float*)(sv + L.rs1);
  const void* qkv = sv + L.qkv;
  const void* O = sv + L.O; const float* lse = (const float*)(sv + L.lse);
  const void* h = sv + L.h; const float* mu2 = (const float*)(sv + L.mu2);
  const float* rs2 = (const float*)(sv + L.rs2);
  const void* c = sv + L.c; const void* u = sv + L.u; const void* m = sv + L.m;
  void* dh = P(scratch, Z.dh); void* p = P(scratch, Z.p); void* du = P(scratch, Z.du);
  void* dr = d.post ? P(scratch, Z.dr) : nullptr;
  void* gm = d.dh1.thr ? P(scratch, Z.gm) : nullptr;
  void* dm = P(scratch, Z.dm); void* dO = P(scratch, Z.dO);
  float* Dbuf = (float*)P(scratch, Z.Dbuf); void* dqkv = P(scratch, Z.dqkv);
  float* part = (float*)P(scratch, Z.part); float* red = (float*)P(scratch, Z.red);
  void* ws = Z.total > Z.ws ? P(scratch, Z.ws) : nullptr;
  const bool all = phase == MTB_PHASE_ALL;
  const bool post = d.post;
  const bool fused = all && !(comm && comm->allreduce);
  // upstream gradient of the MLP branch: dout (pre-LN) or LN2's input
  // gradient dr2 (post-LN, kept in the dh buffer until SEG1)
  const void* G = post ? dh : dout;
  // the MLP branch's own gradient: G through the dropout of the MLP output
  const void* Gm = d.dh2.thr ? gm : G;
  if (all) trace_begin(MTB_TRACE_BWD, st);

  if (phase == MTB_PHASE_ALL || phase == MTB_PHASE_SEG0) {
    if (post) {
      // post-LN: out = LN2(r2), r2 kept in the `a` slot
      MTB_HIP(ln_bwd(dt, T, H, dout, nullptr, a, mu2, rs2, w->ln2_g, nullptr, dh, st));
      if (g.ln2_g) MTB_HIP(colsum(dt, T, H, dout, nullptr, H, a, mu2, rs2, g.ln2_g, red, st));
      if (g.ln2_b) MTB_HIP(colsum(dt, T, H, dout, nullptr, H, nullptr, nullptr, nullptr, g.ln2_b, red, st));
    }
    if (d.dh2.thr) MTB_HIP(drop_apply(dt, (size_t)d.T * d.H, G, gm, d.dh2, st));
    // fc2 backward: dm = G W2 with the activation's derivative fused (bf16)
    if (bf) {
      Epi e;
      e.kind = d.act == MTB_ACT_GELU ? EPI_DGELU : EPI_DSWIGLU;
      e.out = du; e.ldo = Fu; e.aux = u; e.ldaux = Fu; e.ws = ws;
      MTB_HIP(gemm(dt, T, F, H, Gm, H, true, w->w_fc2, F, false, e, st));
    } else {
      Epi e;
      e.out = dm; e.ldo = F;
      MTB_HIP(gemm(dt, T, F, H, Gm, H, true, w->w_fc2, F, false, e, st));
      MTB_HIP(act_bwd(dt, d.act, T, F, dm, u, du, st));
    }
    // the two MLP weight gradients as one grouped launch when both are requested
    if (g.w_fc2 && g.w_fc1) {
      GemmProb p2 = wgrad_fc2(d, Gm, m), p1 = wgrad_fc1(d, du, c);
      p2.e.out = g.w_fc2;
      p1.e.out = g.w_fc1;
      trace_begin(MTB_TRACE_FC2_WGRAD, st);
      MTB_HIP(gemm_wgrad_pair(dt, p2, p1, ws, st));
      trace_end(MTB_TRACE_FC2_WGRAD, st);
    } else if (g.w_fc2) {
      Epi e;
      e.out = g.w_fc2; e.ldo = F; e.ws = ws;
      trace_begin(MTB_TRACE_FC2_WGRAD, st);
      MTB_HIP(gemm(dt, H, F, T, Gm, H, false, m, F, false, e, st));
      trace_end(MTB_TRACE_FC2_WGRAD, st);
    } else if (g.w_fc1) {
      Epi e;
      e.out = g.w_fc1; e.ldo = H; e.ws = ws;
      MTB_HIP(gemm(dt, Fu, H, T, du, Fu, false, c, H, false, e, st));
    }
    if (g.b_fc2) MTB_HIP(colsum(dt, T, H, Gm, nullptr, H, nullptr, nullptr, nullptr, g.b_fc2, red, st));
    if (g.b_fc1) MTB_HIP(colsum(dt, T, Fu, du, nullptr, Fu, nullptr, nullptr, nullptr, g.b_fc1, red, st));
    // fc1 input gradient: partial over ranks, summed at f1
    Epi e;
    e.out = phase == MTB_PHASE_SEG0 ? dx : p; e.ldo = H; e.ws = ws;
    MTB_HIP(gemm(dt, T, H, Fu, du, Fu, true, w->w_fc1, H, false, e, st));
    if (phase == MTB_PHASE_SEG0) return MTB_OK;
    if ((s = call_hook(comm, p, d.T * d.H, dt, MTB_OP_SUM, st)) != MTB_OK) return s;
  }

  if (phase == MTB_PHASE_ALL || phase == MTB_PHASE_SEG1) {
    const void* dc = phase == MTB_PHASE_SEG1 ? reduced_in : p;
    // upstream gradient of the attention branch
    const void* dA;
    if (post) {
      // LN1 backward of the gradient at h = LN1(r1): residual dr2 + MLP input dc
      MTB_HIP(ln_bwd(dt, T, H, dc, dh, h, mu1, rs1, w->ln1_g, nullptr, dr, st));
      if (g.ln1_g) MTB_HIP(colsum(dt, T, H, dc, dh, H, h, mu1, rs1, g.ln1_g, red, st));
      if (g.ln1_b) MTB_HIP(colsum(dt, T, H, dc, dh, H, nullptr, nullptr, nullptr, g.ln1_b, red, st));
      dA = dr;
    } else {
      // LN2 backward + residual: dh = G + LN2^T(dc)
      MTB_HIP(ln_bwd(dt, T, H, dc, nullptr, h, mu2, rs2, w->ln2_g, G, dh, st));
      if (g.ln2_g) MTB_HIP(colsum(dt, T, H, dc, nullptr, H, h, mu2, rs2, g.ln2_g, red, st));
      if (g.ln2_b) MTB_HIP(colsum(dt, T, H, dc, nullptr, H, nullptr, nullptr, nullptr, g.ln2_b, red, st));
      dA = dh;
    }
    // the attention branch's own gradient: through the attention output's dropout
    if (d.dh1.thr) {
      MTB_HIP(drop_apply(dt, (size_t)d.T * d.H, dA, gm, d.dh1, st));
      dA = gm;
    }
    // projection backward (row-parallel: g1's backward is the identity)
    {
      Epi e;
      e.out = dO; e.ldo = NO; e.ws = ws;
      MTB_HIP(gemm(dt, T, NO, H, dA, H, true, w->w_o, NO, false, e, st));
    }
    // the projection's weight gradient waits for the QKV one when both are
    // requested: one grouped launch (gemm_wgrad_pair) after the attention
    const bool wpair = g.w_o && g.w_qkv;
    if (g.w_o && !wpair) {
      Epi e;
      e.out = g.w_o; e.ldo = NO; e.ws = ws;
      MTB_HIP(gemm(dt, H, NO, T, dA, H, false, O, NO, false, e, st));
    }
    if (g.b_o) MTB_HIP(colsum(dt, T, H, dA, nullptr, H, nullptr, nullptr, nullptr, g.b_o, red, st));
    // attention backward
    MTB_HIP(attn_bwd(dt, (int)d.B, S, (int)d.nq, (int)d.nkv, (int)d.d, d.causal, qkv, O, dO, lse, Dbuf,
                     dqkv, part, st, d.dattn));
    if (wpair) {
      GemmProb pq = wgrad_qkv(d, dqkv, post ? x : a), po = wgrad_proj(d, dA, O);
      pq.e.out = g.w_qkv;
      po.e.out = g.w_o;
      MTB_HIP(gemm_wgrad_pair(dt, pq, po, ws, st));
    } else if (g.w_qkv) {
      Epi e;
      e.out = g.w_qkv; e.ldo = H; e.ws = ws;
      MTB_HIP(gemm(dt, Nq, H, T, dqkv, Nq, false, post ? x : a, H, false, e, st));
    }
    if (g.b_qkv) MTB_HIP(colsum(dt, T, Nq, dqkv, nullptr, Nq, nullptr, nullptr, nullptr, g.b_qkv, red, st));
    // QKV input gradient: partial over ranks, summed at f2 (post-LN with the
    // identity reduction: dx = dr1 + da straight from the epilogue)
    Epi e;
    e.out = phase == MTB_PHASE_SEG1 ? dx : p; e.ldo = H; e.ws = ws;
    if (post && fused) {
      e.out = dx; e.resid = dr; e.ldr = H;
    }
    MTB_HIP(gemm(dt, T, H, Nq, dqkv, Nq, true, w->w_qkv, H, false, e, st));
    if (phase == MTB_PHASE_SEG1) return MTB_OK;
    if (post && fused) {
      trace_end(MTB_TRACE_BWD, st);
      return MTB_OK;
    }
    if ((s = call_hook(comm, p, d.T * d.H, dt, MTB_OP_SUM, st)) != MTB_OK) return s;
  }

  const void* da = phase == MTB_PHASE_SEG2 ? reduced_in : p;
  if (post) {
    // the attention read x itself: dx = dr1 + da
    MTB_HIP(add3(dt, T, H, dr, da, nullptr, dx, st));
  } else {
    // LN1 backward + residual: dx = dh + LN1^T(da)
    trace_begin(MTB_TRACE_LN1_BWD, st);
    MTB_HIP(ln_bwd(dt, T, H, da, nullptr, x, mu1, rs1, w->ln1_g, dh, dx, st));
    trace_end(MTB_TRACE_LN1_BWD, st);
    if (g.ln1_g) MTB_HIP(colsum(dt, T, H, da, nullptr, H, x, mu1, rs1, g.ln1_g, red, st));
    if (g.ln1_b) MTB_HIP(colsum(dt, T, H, da, nullptr, H, nullptr, nullptr, nullptr, g.ln1_b, red, st));
  }
  if (all) trace_end(MTB_TRACE_BWD, st);
  return MTB_OK;
}

mtb_status mtb_vocab_xent(int64_t n, int64_t v, int64_t v0, int32_t dtype, int32_t phase,
                          const void* logits, const int64_t* target, float* stats, float* loss,
                          const float* dloss, void* dlogits, const mtb_comm* comm,
                          void* hip_stream) {
  if (n <= 0 || v <= 0 || v0 < 0) return fail(MTB_EINVAL, "n_tokens, v_local must be > 0, v_start >= 0");
  if (n > 0x7fffffff) return fail(MTB_EUNSUPPORTED, "n_tokens beyond 2^31");
  if (dtype != MTB_F32 && dtype != MTB_BF16) return fail(MTB_EINVAL, "bad dtype %d", dtype);
  if (phase < MTB_XENT_PARTIAL || phase > MTB_XENT_ALL) return fail(MTB_EINVAL, "bad phase %d", phase);
  MTB_REQ_A(target, "target", 8);
  MTB_REQ_A(stats, "stats", 4);
  if (phase != MTB_XENT_FINISH || dlogits) MTB_REQ(logits, "logits");
  MTB_OPT_A(loss, "loss", 4);
  MTB_OPT_A(dloss, "dloss", 4);
  MTB_OPT(dlogits, "dlogits");
  if (dlogits && !dloss) return fail(MTB_EINVAL, "dlogits requested without dloss");
  hipStream_t st = (hipStream_t)hip_stream;
  mtb_status s;
  if (phase == MTB_XENT_PARTIAL) {
    MTB_HIP(xent_partial(dtype, n, v, v0, logits, target, stats, nullptr, st));
    return MTB_OK;
  }
  if (phase == MTB_XENT_ALL) {
    const bool hook = comm && comm->allreduce;
    MTB_HIP(xent_partial(dtype, n, v, v0, logits, target, stats, hook ? stats + 3 * n : nullptr, st));
    if (hook) {
      if ((s = call_hook(comm, stats, n, MTB_F32, MTB_OP_MAX, st)) != MTB_OK) return s;
      MTB_HIP(xent_rescale(n, stats, stats + 3 * n, st));
      if ((s = call_hook(comm, stats + n, n, MTB_F32, MTB_OP_SUM, st)) != MTB_OK) return s;
      if ((s = call_hook(comm, stats + 2 * n, n, MTB_F32, MTB_OP_SUM, st)) != MTB_OK) return s;
    }
  }
  if (loss || dlogits)
    MTB_HIP(xent_finish(dtype, n, v, v0, logits, target, stats, loss, dloss, dlogits, st));
  return MTB_OK;
}

mtb_status mtb_vocab_xent_combine(int64_t n, int32_t n_shards, const float* shard_stats,
                                  float* stats, float* loss, void* hip_stream) {
  if (n <= 0 || n_shards <= 0) return fail(MTB_EINVAL, "n_tokens and n_shards must be > 0");
  MTB_REQ_A(shard_stats, "shard_stats", 4);
  MTB_REQ_A(stats, "stats", 4);
  MTB_OPT_A(loss, "loss", 4);
  MTB_HIP(xent_combine(n, n_shards, shard_stats, stats, loss, (hipStream_t)hip_stream));
  return MTB_OK;
}

mtb_status mtb_vocab_embed_fwd(int64_t n, int64_t v, int64_t v0, int64_t h, int32_t dtype,
                               const int64_t* ids, const void* table, void* out,
                               const mtb_comm* comm, void* hip_stream) {
  mtb_status s = check_embed(n, v, v0, h, dtype);
  if (s != MTB_OK) return s;
  MTB_REQ_A(ids, "ids", 8);
  MTB_REQ(table, "table");
  MTB_REQ(out, "out");
  hipStream_t st = (hipStream_t)hip_stream;
  MTB_HIP(embed_fwd(dtype, n, v, v0, (int)h, ids, table, out, st));
  return call_hook(comm, out, n * h, dtype, MTB_OP_SUM, st);
}

size_t mtb_vocab_embed_bwd_workspace_bytes(int64_t n, int64_t v) {
  if (n <= 0 || n > 0x7fffffff || v <= 0 || v > 0x7fffffff) return 0;
  return embed_ws_bytes(v);
}

mtb_status mtb_vocab_embed_bwd(int64_t n, int64_t v, int64_t v0, int64_t h, int32_t dtype,
                               const int64_t* ids, const void* dout, void* dtable,
                               void* workspace, void* hip_stream) {
  mtb_status s = check_embed(n, v, v0, h, dtype);
  if (s != MTB_OK) return s;
  MTB_REQ_A(ids, "ids", 8);
  MTB_REQ(dout, "dout");
  MTB_REQ(dtable, "dtable");
  MTB_REQ(workspace, "workspace");
  MTB_HIP(embed_bwd(dtype, n, v, v0, (int)h, ids, dout, dtable, workspace, (hipStream_t)hip_stream));
  return MTB_OK;
}

mtb_status mtb_vocab_embed_bwd_noalloc(int64_t n, int64_t v, int64_t v0, int64_t h, int32_t dtype,
                                       const int64_t* ids, const void* dout, void* dtable,
                                       void* hip_stream) {
  mtb_status s = check_embed(n, v, v0, h, dtype);
  if (s != MTB_OK) return s;
  if (v > MTB_EMBED_NOALLOC_MAX_ROWS)
    return fail(MTB_EUNSUPPORTED, "v_local %lld exceeds the no-alloc workspace (%d rows)", (long long)v,
                (int)MTB_EMBED_NOALLOC_MAX_ROWS);
  MTB_REQ_A(ids, "ids", 8);
  MTB_REQ(dout, "dout");
  MTB_REQ(dtable, "dtable");
  void* ws = nullptr;
  MTB_HIP(embed_scratch(&ws));
  MTB_HIP(embed_bwd(dtype, n, v, v0, (int)h, ids, dout, dtable, ws, (hipStream_t)hip_stream));
  return MTB_OK;
}

size_t mtb_lmhead_xent_workspace_bytes(int64_t n, int64_t h, int64_t v) {
  if (n <= 0 || h <= 0 || v <= 0 || n > 0x7fffffff || h > 0x7fffffff || v > 0x7fffffff) return 0;
  const size_t parts = (size_t)n * lmhead_tiles(n, h, v) * 3 * sizeof(float);
  const size_t dz = (size_t)n * v * 2;
  return parts > dz ? parts : dz;
}

mtb_status mtb_lmhead_xent_fwd(int64_t n, int64_t h, int64_t v, int64_t v0, int32_t dtype,
                               const void* hid, const void* w, const int64_t* target,
                               float* stats, float* loss, void* logits, void* workspace,
                               const mtb_comm* comm, void* hip_stream) {
  mtb_status s = check_lmhead(n, h, v, v0, dtype);
  if (s != MTB_OK) return s;
  MTB_REQ(hid, "h");
  MTB_REQ(w, "w");
  MTB_REQ_A(target, "target", 8);
  MTB_REQ_A(stats, "stats", 4);
  MTB_OPT_A(loss, "loss", 4);
  MTB_OPT(logits, "logits");
  MTB_REQ(workspace, "workspace");
  hipStream_t st = (hipStream_t)hip_stream;
  // logits tile by tile, reduced in the epilogue; stored only if asked for
  Epi e;
  e.kind = EPI_XENT_STATS;
  e.out = workspace;
  e.out2 = logits;
  e.ldo2 = (int)v;
  e.target = target;
  e.col0 = v0;
  MTB_HIP(gemm(MTB_BF16, (int)n, (int)v, (int)h, hid, (int)h, true, w, (int)h, true, e, st));
  const bool hook = comm && comm->allreduce;
  MTB_HIP(lmhead_combine(n, lmhead_tiles(n, h, v), (const float*)workspace, stats,
                         hook ? stats + 3 * n : nullptr, st));
  if (hook) {
    if ((s = call_hook(comm, stats, n, MTB_F32, MTB_OP_MAX, st)) != MTB_OK) return s;
    MTB_HIP(xent_rescale(n, stats, stats + 3 * n, st));
    if ((s = call_hook(comm, stats + n, n, MTB_F32, MTB_OP_SUM, st)) != MTB_OK) return s;
    if ((s = call_hook(comm, stats + 2 * n, n, MTB_F32, MTB_OP_SUM, st)) != MTB_OK) return s;
  }
  if (loss)
    MTB_HIP(xent_finish(MTB_BF16, n, v, v0, nullptr, target, stats, loss, nullptr, nullptr, st));
  return MTB_OK;
}

mtb_status mtb_lmhead_xent_bwd(int64_t n, int64_t h, int64_t v, int64_t v0, int32_t dtype,
                               const void* hid, const void* w, const int64_t* target,
                               const float* stats, const float* dloss, void* logits, void* dh,
                               void* dw, void* workspace, const mtb_comm* comm,
                               void* hip_stream) {
  mtb_status s = check_lmhead(n, h, v, v0, dtype);
  if (s != MTB_OK) return s;
  MTB_REQ(hid, "h");
  MTB_REQ(w, "w");
  MTB_REQ_A(target, "target", 8);
  MTB_REQ_A(stats, "stats", 4);
  MTB_REQ_A(dloss, "dloss", 4);
  MTB_OPT(dh, "dh");
  MTB_OPT(dw, "dw");
  if (!dh && !dw) return fail(MTB_EINVAL, "neither dh nor dw requested");
  MTB_OPT(logits, "logits");
  if (!logits) MTB_REQ(workspace, "workspace");
  hipStream_t st = (hipStream_t)hip_stream;
  // dz = (softmax - onehot) * dloss, bf16 [n][v]: from the stored logits, in
  // place, or from logits recomputed by a GEMM whose epilogue forms it
  void* dz = logits ? logits : workspace;
  if (logits) {
    MTB_HIP(xent_finish(MTB_BF16, n, v, v0, logits, target, stats, nullptr, dloss, dz, st));
  } else {
    Epi e;
    e.kind = EPI_XENT_GRAD;
    e.out = dz;
    e.ldo = (int)v;
    e.target = target;
    e.col0 = v0;
    e.rowstat = stats;
    e.rowscale = dloss;
    MTB_HIP(gemm(MTB_BF16, (int)n, (int)v, (int)h, hid, (int)h, true, w, (int)h, true, e, st));
  }
  if (dw) {  // dW = dz^T h: both operands token-major
    Epi e;
    e.out = dw;
    e.ldo = (int)h;
    MTB_HIP(gemm(MTB_BF16, (int)v, (int)h, (int)n, dz, (int)v, false, hid, (int)h, false, e, st));
  }
  if (dh) {  // dh = dz W: this shard's partial of the column-parallel input's gradient
    Epi e;
    e.out = dh;
    e.ldo = (int)h;
    MTB_HIP(gemm(MTB_BF16, (int)n, (int)h, (int)v, dz, (int)v, true, w, (int)h, false, e, st));
    if ((s = call_hook(comm, dh, n * h, MTB_BF16, MTB_OP_SUM, st)) != MTB_OK) return s;
  }
  return MTB_OK;
}

}  // extern "C"
