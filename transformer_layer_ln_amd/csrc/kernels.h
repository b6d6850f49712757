// Host-side launchers of the gfx950 kernels (internal to libmtb).
// dtype is MTB_F32 (0) or MTB_BF16 (1) as in mtb.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtb {

// Dropout of one site ([TP-block] sec. 5): a counter-based mask, a pure
// function of (key, site, offset, flat element index i): the 32-bit word
// i & 3 of Philox4x32-10(counter = (i >> 2 as two 32-bit words, site,
// offset), key); the element is dropped when that word is below thr, and a
// kept element is scaled by `scale` = 1 / (1 - p).
struct Drop {
  uint32_t thr = 0;          // floor(p * 2^32); 0: no dropout at this site
  float scale = 1.0f;
  uint32_t k0 = 0, k1 = 0;   // seed, low and high 32 bits
  uint32_t site = 0, offset = 0;
};

// GEMM epilogues. The product is C[m][n] = sum_k A(m,k) B(n,k).
enum EpiKind {
  EPI_STORE = 0,    // out = C (+bias[n]) (+resid[m][n])
  EPI_GELU = 1,     // u = C (+bias): out = u, out2 = GELU(u)
  EPI_SWIGLU = 2,   // u = C (+bias) over interleaved gate/up columns: out = u [M][2F],
                    // out2[m][f] = silu(gate) * up  [M][F]
  EPI_DGELU = 3,    // out = C * GELU'(aux[m][n])
  EPI_DSWIGLU = 4,  // C = dm [M][F]; aux = u [M][2F] interleaved: out [M][2F] = (d gate, d up)
  EPI_XENT_STATS = 5,  // C = logits [M][N] (vocab columns from col0): per row and BN-wide column
                       // tile, (max, sum exp(C - max), C at the row's target or 0) to
                       // out (float) [M][tiles_n][3]; with out2 the logits are also stored
                       // (bf16 [M][ldo2]) and the statistics are those of the stored values
  EPI_XENT_GRAD = 6,   // out = (exp(C - M_r) / S_r - [col0 + n == target_r]) * dloss_r with
                       // M_r = rowstat[r], S_r = rowstat[M + r], dloss_r = rowscale[r]
};

struct Epi {
  int kind = EPI_STORE;
  void* out = nullptr;         // [M][ldo]
  int ldo = 0;
  void* out2 = nullptr;        // [M][ldo2]
  int ldo2 = 0;
  const void* bias = nullptr;  // [N]
  const void* resid = nullptr; // [M][ldr]
  int ldr = 0;
  const void* aux = nullptr;   // [M][ldaux]
  int ldaux = 0;
  void* ws = nullptr;          // fp32 workspace for split-K partial tiles (gemm_ws_bytes), or null
  const int64_t* target = nullptr;  // EPI_XENT_*: [M] global target ids
  int64_t col0 = 0;                 // EPI_XENT_*: global vocab id of column 0
  const float* rowstat = nullptr;   // EPI_XENT_GRAD: [2][M] (max, sum exp)
  const float* rowscale = nullptr;  // EPI_XENT_GRAD: [M] loss cotangent
  Drop drop;                   // EPI_STORE: out = resid + dropout(C + bias), element index
                               // m * N + n (the [T][H] hidden state)
};

// C = A . B^T-style product with operand majorness:
//   a_kc: A stored [M][K] (k contiguous) else [K][M];
//   b_kc: B stored [N][K] (k contiguous) else [K][N].
hipError_t gemm(int dtype, int M, int N, int K, const void* A, int lda, bool a_kc,
                const void* B, int ldb, bool b_kc, const Epi& e, hipStream_t st);
// Bytes of Epi::ws that gemm() uses to split the contraction of this product
// over several workgroups per output tile (0: it does not split). Plain-store
// products (weight gradients; token-major products) with too few tiles to
// fill the chip are split; the partial tiles are summed in a fixed order.
size_t gemm_ws_bytes(int dtype, int M, int N, int K, bool a_kc, bool b_kc, int kind);
// One product for gemm_wgrad_pair: C[M][N] = sum_k A[k][M] B[k][N] (both
// operands stored k-major, as weight gradients read activations), plain store
// to e.out [M][e.ldo] (other Epi fields unused).
struct GemmProb {
  int M, N, K;
  const void* A;
  int lda;
  const void* B;
  int ldb;
  Epi e;
};
// Two independent weight gradients. When their blocks fill the chip together
// -- both contractions split (partial tiles summed in a fixed order), or both
// whole -- and a per-wave cost model favours it, they run in one grid of the
// scheduled kernel; otherwise one after the other, as gemm() runs them. ws:
// gemm_wgrad_pair_ws_bytes bytes.
hipError_t gemm_wgrad_pair(int dtype, const GemmProb& p0, const GemmProb& p1, void* ws, hipStream_t st);
size_t gemm_wgrad_pair_ws_bytes(int dtype, const GemmProb& p0, const GemmProb& p1);
// Column-tile width the bf16 GEMM uses for this problem (the tiles_n of
// EPI_XENT_STATS is ceil(N / it)).
int gemm_tile_n(int M, int N, int K, bool a_kc, bool b_kc, int kind);

// LayerNorm over rows of width H: hsum = x + dropout((resid) (+bias)) rounded
// to dtype (element index row * H + col); y = (hsum - mu) * rstd (* g + b).
// h_out (optional) receives hsum.
hipError_t ln_fwd(int dtype, int rows, int H, const void* x, const void* resid, const void* bias,
                  const void* g, const void* b, void* h_out, void* y, float* mu, float* rstd,
                  float eps, hipStream_t st, const Drop& drop = Drop());
// dx = dres + LN backward of (dy + dy2) at xhat = (hin - mu) * rstd, gain g;
// dy2, dres, g optional.
hipError_t ln_bwd(int dtype, int rows, int H, const void* dy, const void* dy2, const void* hin,
                  const float* mu, const float* rstd, const void* g, const void* dres, void* dx,
                  hipStream_t st);
// column sums over rows: out[n] = sum_r (y + y2)[r][n] (*xhat[r][n] if hin != NULL), written
// in dtype; y2 optional, same leading dimension. part: rows_split * N floats of scratch.
hipError_t colsum(int dtype, int rows, int N, const void* y, const void* y2, int ldy,
                  const void* hin, const float* mu, const float* rstd, void* out, float* part,
                  hipStream_t st);
// number of row splits colsum uses for `rows` rows (part holds splits * N floats)
int colsum_splits(int rows);
// out = a + dropout(b (+bias[n])) elementwise over [rows][H]
hipError_t add3(int dtype, int rows, int H, const void* a, const void* b, const void* bias,
                void* out, hipStream_t st, const Drop& drop = Drop());
// out = in * dropout multiplier over n elements (n % 8 == 0; element index from 0)
hipError_t drop_apply(int dtype, size_t n, const void* in, void* out, const Drop& drop,
                      hipStream_t st);
// activation forward / backward as separate passes (fp32 path)
hipError_t act_fwd(int dtype, int act, int rows, int F, const void* u, void* m, hipStream_t st);
hipError_t act_bwd(int dtype, int act, int rows, int F, const void* dm, const void* u, void* du,
                   hipStream_t st);

// Attention. qkv [T][Nqkv] token-major ([Q heads | K heads | V heads]);
// O [T][nq*d]; lse [B][nq][S] (natural log).
hipError_t attn_fwd(int dtype, int B, int S, int nq, int nkv, int d, int causal, const void* qkv,
                    void* O, float* lse, hipStream_t st, const Drop& drop = Drop());
// dO [T][nq*d]; Dbuf [B][nq][S] fp32 scratch (rowsum(dO o O) per query, formed
// inside the backward); dqkv [T][Nqkv] output; part: fp32 scratch of
// B*nq*S*2*d floats (GQA, bf16).
hipError_t attn_bwd(int dtype, int B, int S, int nq, int nkv, int d, int causal, const void* qkv,
                    const void* O, const void* dO, const float* lse, float* Dbuf, void* dqkv,
                    float* part, hipStream_t st, const Drop& drop = Drop());

// Vocab-sharded cross-entropy.
hipError_t xent_partial(int dtype, int64_t n, int64_t v, int64_t v0, const void* z,
                        const int64_t* tgt, float* stats, float* mloc, hipStream_t st);
hipError_t xent_rescale(int64_t n, float* stats, const float* mloc, hipStream_t st);
hipError_t xent_combine(int64_t n, int R, const float* shard_stats, float* stats, float* loss,
                        hipStream_t st);
hipError_t xent_finish(int dtype, int64_t n, int64_t v, int64_t v0, const void* z,
                       const int64_t* tgt, const float* stats, float* loss, const float* dloss,
                       void* dz, hipStream_t st);

// LM head: merge per-column-tile logits statistics [n][tiles][3] into [3][n].
hipError_t lmhead_combine(int64_t n, int tiles, const float* parts, float* stats, float* mloc,
                          hipStream_t st);

// Vocab-parallel embedding (one vocab shard [v0, v0 + vl) of the table).
// Backward workspace: per table row, an int32 token count and first token.
size_t embed_ws_bytes(int64_t vl);
// the library's own backward workspace on the current device (a file-scope
// device array of MTB_EMBED_NOALLOC_MAX_ROWS rows; see embed.hip)
hipError_t embed_scratch(void** ptr);
hipError_t embed_fwd(int dtype, int64_t n, int64_t vl, int64_t v0, int H, const int64_t* ids,
                     const void* table, void* out, hipStream_t st);
hipError_t embed_bwd(int dtype, int64_t n, int64_t vl, int64_t v0, int H, const int64_t* ids,
                     const void* dout, void* dtable, void* workspace, hipStream_t st);

}  // namespace mtb
