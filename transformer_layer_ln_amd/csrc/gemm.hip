// GEMMs of the block: C[m][n] = sum_k A(m,k) B(n,k) with fused epilogues.
//
// bf16 path, gfx950 MFMA v_mfma_f32_32x32x16_bf16, two kernels:
//  * gemm_bf16_sched_kernel (contractions >= 1024 deep, multiples of 32): a
//    256 x 256 tile on 8 wavefronts of 128 x 64 (two per SIMD; a 256 x 192
//    tile on 4 wavefronts for 1536-wide products), its k-loop one hand-scheduled
//    inline-assembly block (gemm_loop.inc, written by gen_gemm_loop.py, which
//    describes the schedule): direct-to-LDS copies three 32-deep k-tiles
//    ahead, fragments read a whole k-tile before their MFMAs;
//  * gemm_bf16_kernel (the other shapes): a grid of 2x2, 2x4 or 4x2
//    wavefronts per block, block tile BM x BN x 64, LDS double-buffered (one
//    barrier per k-step: the next tile is fetched into registers while the
//    current one is multiplied, then written to the other LDS buffer).
// In both, a k-contiguous operand sits in LDS as [row][k] with 16-byte chunks
// XOR-swizzled by row, so a fragment is one ds_read_b128 per lane. An operand
// whose contraction index is not the contiguous one (dgrad's weight, both
// wgrad operands) is copied as it is, [k][row], and its fragments come from
// two LDS transpose reads (ds_read_b64_tr_b16) per lane: no register
// transposes (measured 6 % faster on the weight gradients than transposing in
// registers on the way to LDS).
//
// The MFMA is issued as (B-fragment, A-fragment), i.e. it computes C^T, so
// that each lane ends up holding 4 consecutive n of one row m.
//
// Epilogue: the fp32 accumulator tile is staged in LDS (a chunk of rows at a
// time, reusing the operand buffers) and then read back row-wise, so that
// every global access of the epilogue -- bias, residual and derivative
// inputs, the stored outputs -- is 16 bytes per lane over whole rows. Storing
// straight from the MFMA layout touches 32 rows per instruction with 16 bytes
// each; on MI355X those partial-line writes reach HBM several times over
// (measured 3.5x the output bytes for the two-output GELU epilogue).
//
// Uses in the block ([TP-block] sec. 1-2; [MLM-notes] Column/RowParallelLinear):
//   forward   Y = X W^T         A = X [T][in],  B = W [out][in]     (k-contig both)
//   dgrad     dX = dY W         A = dY [T][out], B = W [out][in]    (B transposed)
//   wgrad     dW = dY^T X       A = dY [T][out], B = X [T][in]      (both transposed)
#include <algorithm>
#include <type_traits>

#include "drop.h"
#include "gemm_loop.inc"

#include "common.h"
#include "kernels.h"

namespace mtb {
namespace {

constexpr int BK = 64;
constexpr int EPI_PARTIAL = 100;  // internal: fp32 partial tile of a split contraction

MTB_DEV int swz(int row) { return (row ^ (row >> 3)) & 7; }

// operand tile ROWS x BK from a matrix stored [rows][K] (k contiguous),
// NT threads, 16-byte chunks (threads past the last chunk idle)
template <int ROWS, int NT>
struct TileKc {
  static constexpr int TOT = ROWS * BK / 8;
  static constexpr int NCH = (TOT + NT - 1) / NT;
  u32x4 r[NCH];
  MTB_DEV void load(const bf16_t* __restrict__ p, int ld, int row0, int rowmax, int k0, int kmax,
                    int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + NT * i, row = q >> 3, c = q & 7;
      if (TOT % NT != 0 && q >= TOT) break;
      const int gr = min(row0 + row, rowmax - 1);
      // past the contraction's end (K % 64 != 0): zeros
      r[i] = k0 + c * 8 < kmax ? *reinterpret_cast<const u32x4*>(p + (size_t)gr * ld + k0 + c * 8)
                               : u32x4{0u, 0u, 0u, 0u};
    }
  }
  MTB_DEV void store(bf16_t* s, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + NT * i, row = q >> 3, c = q & 7;
      if (TOT % NT != 0 && q >= TOT) break;
      *reinterpret_cast<u32x4*>(s + row * BK + ((c ^ swz(row)) << 3)) = r[i];
    }
  }
};

// operand tile ROWS x BK from a matrix stored [K][rows] (rows contiguous),
// kept in that layout in LDS: [BK][ROWS], 16-byte chunks of a k row permuted
// by chunk ^ 4 (k mod 4). The MFMA fragments are read with the LDS transpose
// read (64 bits per lane: within each 16-lane group, lane i receives element
// i mod 4 of the 8 bytes addressed by lanes 4j + i / 4, j = 0..3), so the
// tile is copied as it is and never transposed in registers.
MTB_DEV int swt(int k) { return (k & 3) << 2; }

template <int ROWS, int NT>
struct TileMnT {
  static_assert(ROWS == 128 || ROWS == 256, "chunk permutation needs 16 or 32 chunks per row");
  static constexpr int CPR = ROWS / 8;  // 16-byte chunks per k row
  static constexpr int TOT = BK * CPR;
  static constexpr int NCH = (TOT + NT - 1) / NT;
  u32x4 r[NCH];
  MTB_DEV void load(const bf16_t* __restrict__ p, int ld, int row0, int rowmax, int k0, int kmax,
                    int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + NT * i, k = q / CPR, c = q % CPR;
      if (TOT % NT != 0 && q >= TOT) break;
      const int gm = min(row0 + c * 8, rowmax - 8);
      // past the contraction's end: zeros
      r[i] = k0 + k < kmax ? *reinterpret_cast<const u32x4*>(p + (size_t)(k0 + k) * ld + gm)
                           : u32x4{0u, 0u, 0u, 0u};
    }
  }
  MTB_DEV void store(bf16_t* s, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int q = tid + NT * i, k = q / CPR, c = q % CPR;
      if (TOT % NT != 0 && q >= TOT) break;
      *reinterpret_cast<u32x4*>(s + k * ROWS + ((c ^ swt(k)) << 3)) = r[i];
    }
  }
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_t;

// MFMA fragment (rows r0 .. r0+31, k = 16 kk .. 16 kk + 15; lane: row r0 + lane % 32,
// k 8 (lane / 32) .. +7) of a [BK][ROWS] tile: two transpose reads of 4 k each
template <int ROWS>
MTB_DEV bf16x8 frag_tr(const bf16_t* s, int r0, int kk, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int m = r0 + 16 * (g & 1) + 4 * (sl & 3);
  const int k = kk * 16 + 8 * (g >> 1) + (sl >> 2);
  const int off = ((m >> 3) ^ swt(k)) * 8 + (m & 7);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)(s + k * ROWS + off));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t)(s + (k + 4) * ROWS + off));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

template <typename T>
MTB_DEV void ld4g(const void* p, size_t off, float (&v)[4]) {
  ld4(reinterpret_cast<const T*>(p) + off, v);
}

// fp32 path epilogue (plain store, optional bias and residual) for 4
// consecutive columns n..n+3 of row m
MTB_DEV void epi4_f32(const Epi& e, int m, int n, int N, float (&v)[4]) {
  if (e.bias) {
    float b[4];
    ld4g<float>(e.bias, n, b);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += b[r];
  }
  if (e.drop.thr) {  // dropout of (C + bias) before the residual add
    float k[4];
    drop_mul4(e.drop, ((uint64_t)m * N + n) >> 2, k);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] *= k[r];
  }
  if (e.resid) {
    float b[4];
    ld4g<float>(e.resid, (size_t)m * e.ldr + n, b);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] += b[r];
  }
  st4(reinterpret_cast<float*>(e.out) + (size_t)m * e.ldo + n, v);
}

// 8 bf16 values at p + off -> floats, added to v
MTB_DEV void add8(const void* p, size_t off, float (&v)[8]) {
  float b[8];
  ld8(reinterpret_cast<const bf16_t*>(p) + off, b);
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] += b[r];
}
MTB_DEV void out8(void* p, size_t off, const float (&v)[8]) {
  st8(reinterpret_cast<bf16_t*>(p) + off, v);
}

// rows of the tile staged per epilogue chunk: the largest multiple of the
// wavefront tile height wm that divides bm and fits the operand buffers
// (max_rows = their size in fp32 rows)
constexpr int stage_rows(int bm, int wm, int max_rows, int c) {
  return c <= wm ? wm : (bm % c == 0 && c <= max_rows ? c : stage_rows(bm, wm, max_rows, c - wm));
}

// Staged fp32 tile: CR rows x BN columns, 16-byte chunks XOR-swizzled by row.
template <int BN>
struct Staged {
  static constexpr int NCH = BN / 4;      // 16-byte chunks per row
  static constexpr int G = NCH & -NCH;    // XOR-swizzle within aligned groups of G chunks
  float* s;
  MTB_DEV int off(int r, int n) const {
    const int c = n >> 2;
    return r * BN + (((c & ~(G - 1)) | ((c ^ r) & (G - 1))) << 2) + (n & 3);
  }
  MTB_DEV void put4(int r, int n, const f32x4& v) const { *reinterpret_cast<f32x4*>(s + off(r, n)) = v; }
  MTB_DEV void get8(int r, int n, float (&v)[8]) const {
    const f32x4 a = *reinterpret_cast<const f32x4*>(s + off(r, n));
    const f32x4 b = *reinterpret_cast<const f32x4*>(s + off(r, n + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  MTB_DEV float get(int r, int n) const { return s[off(r, n)]; }
};

// One bf16 operand of a staged chunk's row phase (the residual of EPI_STORE,
// u of EPI_DGELU), loaded into registers before the chunk's stores: one
// 16-byte load per row item of the row phase (same item order), all in
// flight at once. Loaded one item at a time between the staged reads and the
// stores, the residual cost the seq-2048 fc2 forward about 3x its HBM time (a
// load latency per item).
template <int BN, int CR, int NT>
struct RowOperand {
  static constexpr int IPR = BN / 8, ITEMS = CR * IPR / NT;
  static_assert(CR * IPR % NT == 0, "whole row items per thread");
  u32x4 q[ITEMS];
  MTB_DEV void load(const void* src, int ld, int M, int N, int mc, int n0, int tid) {
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
      const int it = tid + j * NT, r = it / IPR, nl = (it % IPR) * 8;
      const int m = mc + r, n = n0 + nl;
      q[j] = u32x4{0u, 0u, 0u, 0u};
      if (m < M && n < N)
        q[j] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(src) + (size_t)m * ld + n);
    }
  }
};

// Row phase of the epilogue for rows [0, CR) of the staged chunk whose first
// row is global row mc: each work item is 8 consecutive columns of one row
// (for SwiGLU, the 8 gate and the matching 8 up columns).
template <int EPI, int BN, int CR, int NT>
MTB_DEV void epi_rows(const Epi& e, const Staged<BN>& st, int M, int N, int mc, int n0, int tid) {
  if constexpr (EPI == EPI_SWIGLU) {
    // columns 32k..32k+15 are gate features 16k.., 32k+16..32k+31 the matching up features
    constexpr int IPR = BN / 16;
    for (int it = tid; it < CR * IPR; it += NT) {
      const int r = it / IPR, c = it % IPR;
      const int m = mc + r, nl = (c >> 1) * 32 + (c & 1) * 8, n = n0 + nl;
      if (m >= M || n >= N) continue;
      float g[8], u[8], o[8];
      st.get8(r, nl, g);
      st.get8(r, nl + 16, u);
      if (e.bias) {
        add8(e.bias, n, g);
        add8(e.bias, n + 16, u);
      }
      // keep the stored pre-activations and the activation consistent
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        g[i] = bf2f(f2bf(g[i]));
        u[i] = bf2f(f2bf(u[i]));
        o[i] = g[i] * sigmoid_f(g[i]) * u[i];
      }
      const size_t ro = (size_t)m * e.ldo;
      out8(e.out, ro + n, g);
      out8(e.out, ro + n + 16, u);
      out8(e.out2, (size_t)m * e.ldo2 + (n >> 5) * 16 + (n & 15), o);
    }
  } else {
    constexpr int IPR = BN / 8;
    for (int it = tid; it < CR * IPR; it += NT) {
      const int r = it / IPR, nl = (it % IPR) * 8;
      const int m = mc + r, n = n0 + nl;
      if (m >= M || n >= N) continue;
      float v[8];
      st.get8(r, nl, v);
      if constexpr (EPI == EPI_STORE) {
        if (e.bias) add8(e.bias, n, v);
        if (e.drop.thr) drop_apply8(e.drop, (uint64_t)m * N + n, v);
        if (e.resid) add8(e.resid, (size_t)m * e.ldr + n, v);
        out8(e.out, (size_t)m * e.ldo + n, v);
      } else if constexpr (EPI == EPI_GELU) {
        if (e.bias) add8(e.bias, n, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf2f(f2bf(v[i]));
        out8(e.out, (size_t)m * e.ldo + n, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = gelu_f(v[i]);
        out8(e.out2, (size_t)m * e.ldo2 + n, v);
      } else if constexpr (EPI == EPI_DGELU) {
        float u[8];
        ld8(reinterpret_cast<const bf16_t*>(e.aux) + (size_t)m * e.ldaux + n, u);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] *= gelu_grad_f(u[i]);
        out8(e.out, (size_t)m * e.ldo + n, v);
      } else if constexpr (EPI == EPI_DSWIGLU) {
        // v = dm at features n..n+7; their gate/up columns in the interleaved layout
        const int gp = (n >> 4) * 32 + (n & 15);
        float ug[8], uu[8], dg[8], du[8];
        ld8(reinterpret_cast<const bf16_t*>(e.aux) + (size_t)m * e.ldaux + gp, ug);
        ld8(reinterpret_cast<const bf16_t*>(e.aux) + (size_t)m * e.ldaux + gp + 16, uu);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float sg = sigmoid_f(ug[i]);
          dg[i] = v[i] * uu[i] * sg * (1.0f + ug[i] * (1.0f - sg));
          du[i] = v[i] * ug[i] * sg;
        }
        out8(e.out, (size_t)m * e.ldo + gp, dg);
        out8(e.out, (size_t)m * e.ldo + gp + 16, du);
      } else if constexpr (EPI == EPI_XENT_GRAD) {
        // dz = softmax - onehot(target), scaled by the token's loss cotangent
        const float Mx = e.rowstat[m], sc = e.rowscale[m] / e.rowstat[M + m];
        const int64_t lt = e.target[m] - e.col0 - n;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = exp_fast(v[i] - Mx) * sc;
        if (lt >= 0 && lt < 8) v[lt] -= e.rowscale[m];
        out8(e.out, (size_t)m * e.ldo + n, v);
      }
    }
  }
}

// EPI_DSWIGLU's saved gate and up pre-activations for half of a staged
// chunk's row items (same item order as epi_rows), loaded before that half's
// stores; the whole chunk's would take twice the registers.
template <int BN, int CR, int NT>
struct SwiRows {
  static constexpr int IPR = BN / 8, ITEMS = CR * IPR / NT, HALF = ITEMS / 2;
  static_assert(CR * IPR % NT == 0 && ITEMS % 2 == 0, "two halves of whole row items per thread");
  u32x4 g[HALF], u[HALF];
  MTB_DEV void load(const Epi& e, int M, int N, int mc, int n0, int tid, int half) {
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int it = tid + (half * HALF + j) * NT, r = it / IPR, nl = (it % IPR) * 8;
      const int m = mc + r, n = n0 + nl;
      g[j] = u32x4{0u, 0u, 0u, 0u};
      u[j] = g[j];
      if (m < M && n < N) {
        const bf16_t* q = reinterpret_cast<const bf16_t*>(e.aux) + (size_t)m * e.ldaux + (n >> 4) * 32 + (n & 15);
        g[j] = *reinterpret_cast<const u32x4*>(q);
        u[j] = *reinterpret_cast<const u32x4*>(q + 16);
      }
    }
  }
};

// Row phase of EPI_DSWIGLU with the pre-activations prefetched: pre holds the
// first half of the chunk's items on entry; the second half is requested
// after the first half's stores.
template <int BN, int CR, int NT>
MTB_DEV void epi_rows_dswiglu_pre(const Epi& e, const Staged<BN>& st, int M, int N, int mc, int n0,
                                  int tid, SwiRows<BN, CR, NT>& pre) {
  constexpr int IPR = BN / 8, HALF = SwiRows<BN, CR, NT>::HALF;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h == 1) pre.load(e, M, N, mc, n0, tid, 1);
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      const int it = tid + (h * HALF + j) * NT, r = it / IPR, nl = (it % IPR) * 8;
      const int m = mc + r, n = n0 + nl;
      if (m >= M || n >= N) continue;
      float v[8], dg[8], du[8];
      st.get8(r, nl, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t gw = pre.g[j][i >> 1], uw = pre.u[j][i >> 1];
        const float ug = (i & 1) ? hi_f(gw) : lo_f(gw), uu = (i & 1) ? hi_f(uw) : lo_f(uw);
        const float sg = sigmoid_f(ug);
        dg[i] = v[i] * uu * sg * (1.0f + ug * (1.0f - sg));
        du[i] = v[i] * ug * sg;
      }
      const int gp = (n >> 4) * 32 + (n & 15);
      out8(e.out, (size_t)m * e.ldo + gp, dg);
      out8(e.out, (size_t)m * e.ldo + gp + 16, du);
    }
  }
}

// Row phase of a plain store (residual) or EPI_DGELU (u) with that operand
// prefetched (pre): the same items and arithmetic as epi_rows, item j of this
// thread taking pre.q[j].
template <int EPI, int BN, int CR, int NT>
MTB_DEV void epi_rows_pre(const Epi& e, const Staged<BN>& st, int M, int N, int mc, int n0, int tid,
                          const RowOperand<BN, CR, NT>& pre) {
  static_assert(EPI == EPI_STORE || EPI == EPI_DGELU, "prefetched row operand");
  constexpr int IPR = BN / 8, ITEMS = CR * IPR / NT;
#pragma unroll
  for (int j = 0; j < ITEMS; ++j) {
    const int it = tid + j * NT, r = it / IPR, nl = (it % IPR) * 8;
    const int m = mc + r, n = n0 + nl;
    if (m >= M || n >= N) continue;
    float v[8];
    st.get8(r, nl, v);
    if constexpr (EPI == EPI_STORE) {
      if (e.bias) add8(e.bias, n, v);
      if (e.drop.thr) drop_apply8(e.drop, (uint64_t)m * N + n, v);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] += lo_f(pre.q[j][i]);
        v[2 * i + 1] += hi_f(pre.q[j][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] *= gelu_grad_f(lo_f(pre.q[j][i]));
        v[2 * i + 1] *= gelu_grad_f(hi_f(pre.q[j][i]));
      }
    }
    out8(e.out, (size_t)m * e.ldo + n, v);
  }
}

// Row statistics of a logits tile for the vocab cross-entropy: per row of
// the staged chunk, over this tile's valid columns, (max, sum exp(z - max),
// z at the row's target or 0) into out [M][tiles_n][3]. NT / CR threads per
// row, each over a contiguous run of columns, merged by lane shuffles. With
// out2 the logits are also stored (bf16 [M][ldo2]) and the statistics taken
// from those stored values.
template <int BN, int CR, int NT>
MTB_DEV void epi_xent_stats(const Epi& e, const Staged<BN>& st, int M, int N, int mc, int n0, int tn,
                            int tiles_n, int tid) {
  constexpr int TPR = NT / CR, CPT = BN / TPR;
  static_assert(TPR * CR == NT && TPR <= 64 && (TPR & (TPR - 1)) == 0, "threads per row");
  const int r = tid / TPR, part = tid % TPR, m = mc + r;
  const int c0 = part * CPT, cend = min(CPT, N - n0 - c0);   // valid columns of this run
  float mx = -__builtin_huge_valf(), sum = 0.f, tz = 0.f;
  int64_t lt = -1;
  if (m < M) lt = e.target[m] - e.col0 - n0 - c0;
  const bool keep = e.out2 != nullptr;
  auto z = [&](int c) {
    const float v = st.get(r, c0 + c);
    return keep ? bf2f(f2bf(v)) : v;
  };
  if (keep && m < M) {
    static_assert(CPT % 8 == 0, "stored logits go out 8 at a time");
    for (int c = 0; c < cend; c += 8) {  // cend is a multiple of 8 (N % 8 == 0)
      float v[8];
      st.get8(r, c0 + c, v);
      out8(e.out2, (size_t)m * e.ldo2 + n0 + c0 + c, v);
    }
  }
  for (int c = 0; c < cend; ++c) mx = fmaxf(mx, z(c));
  for (int c = 0; c < cend; ++c) sum += exp_fast(z(c) - mx);
  if (lt >= 0 && lt < cend) tz = z((int)lt);
#pragma unroll
  for (int o = 1; o < TPR; o <<= 1) {
    const float m2 = __shfl_xor(mx, o, 64), s2 = __shfl_xor(sum, o, 64);
    tz += __shfl_xor(tz, o, 64);
    const float Mx = fmaxf(mx, m2);
    sum = (mx == -__builtin_huge_valf() ? 0.f : sum * exp_fast(mx - Mx)) +
          (m2 == -__builtin_huge_valf() ? 0.f : s2 * exp_fast(m2 - Mx));
    mx = Mx;
  }
  if (part == 0 && m < M) {
    float* o = reinterpret_cast<float*>(e.out) + ((size_t)m * tiles_n + tn) * 3;
    o[0] = mx;
    o[1] = sum;
    o[2] = tz;
  }
}

// Row phase of a split contraction: the fp32 partial tile to ws [M][N]
template <int BN, int CR, int NT>
MTB_DEV void epi_partial(float* ws, const Staged<BN>& st, int M, int N, int mc, int n0, int tid) {
  constexpr int IPR = BN / 8;
  for (int it = tid; it < CR * IPR; it += NT) {
    const int r = it / IPR, nl = (it % IPR) * 8;
    const int m = mc + r, n = n0 + nl;
    if (m >= M || n >= N) continue;
    float v[8];
    st.get8(r, nl, v);
    st8(ws + (size_t)m * N + n, v);
  }
}

// out[m][n] = sum over s = 0 .. splits-1 of ws[s][m][n], rounded once; 8
// elements per thread (N % 8 == 0)
MTB_DEV void splitk_reduce_at(size_t blk, int M, int N, int splits, const float* __restrict__ ws,
                              bf16_t* __restrict__ out, int ldo) {
  const size_t i = (blk * 256 + threadIdx.x) * 8;
  const size_t MN = (size_t)M * N;
  if (i >= MN) return;
  float v[8];
  ld8(ws + i, v);
  for (int s = 1; s < splits; ++s) {
    float w[8];
    ld8(ws + (size_t)s * MN + i, w);
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] += w[r];
  }
  const size_t m = i / N, n = i % N;
  st8(out + m * ldo + n, v);
}
__global__ __launch_bounds__(256) void splitk_reduce_kernel(int M, int N, int splits,
                                                            const float* __restrict__ ws,
                                                            bf16_t* __restrict__ out, int ldo) {
  splitk_reduce_at(blockIdx.x, M, N, splits, ws, out, ldo);
}
// The split sums of two products in one launch: blocks [0, blocks0) take the
// first, the rest the second (a launch of its own costs more than the few MB
// of a small product's partials take to read).
struct SplitSum {
  int M, N, splits;
  const float* ws;
  bf16_t* out;
  int ldo;
};
__global__ __launch_bounds__(256) void splitk_reduce_pair_kernel(SplitSum a, SplitSum b, int blocks0) {
  const bool second = (int)blockIdx.x >= blocks0;
  const SplitSum& p = second ? b : a;
  splitk_reduce_at(second ? blockIdx.x - blocks0 : blockIdx.x, p.M, p.N, p.splits, p.ws, p.out, p.ldo);
}

// Epilogue of a split contraction with a fused epilogue: sums the fp32
// partial tiles of ws [splits][M][N] in split order into the staged tile, then
// runs the same row (and column) phases as the GEMM kernel. One block per
// BM x BN output tile.
template <int BM, int BN, int NT, int EPI>
__global__ __launch_bounds__(NT) void splitk_epi_kernel(int M, int N, int splits,
                                                        const float* __restrict__ ws, Epi ep) {
  constexpr int CR = BM * BN * 4 <= 65536 ? BM : 65536 / (BN * 4);
  static_assert(BM % CR == 0 && CR % 64 == 0, "staging chunk");
  __shared__ __attribute__((aligned(16))) float smem[CR * BN];
  const Staged<BN> st{smem};
  const int tid = threadIdx.x, tiles_n = (N + BN - 1) / BN;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
  const size_t MN = (size_t)M * N;
  for (int c0 = 0; c0 < BM; c0 += CR) {
    if (c0 > 0) __syncthreads();
    for (int it = tid; it < CR * BN / 8; it += NT) {
      const int r = it / (BN / 8), nl = (it % (BN / 8)) * 8;
      const int m = m0 + c0 + r, n = n0 + nl;
      float v[8] = {};
      if (m < M && n < N) {
        const float* p = ws + (size_t)m * N + n;
        for (int sp = 0; sp < splits; ++sp) {
          float w[8];
          ld8(p + sp * MN, w);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] += w[q];
        }
      }
      st.put4(r, nl, f32x4{v[0], v[1], v[2], v[3]});
      st.put4(r, nl + 4, f32x4{v[4], v[5], v[6], v[7]});
    }
    __syncthreads();
    epi_rows<EPI, BN, CR, NT>(ep, st, M, N, m0 + c0, n0, tid);
  }
}

// Block -> (tile row, tile column, contraction split). Blocks i, i+8, i+16,
// ... share an XCD (and its L2), so each XCD gets a contiguous run of tiles,
// walked GROUP tile-rows at a time so that concurrently running tiles share A
// and B panels. Split s of the contraction takes blocks [s * tiles, (s + 1) *
// tiles).
struct BlockTile {
  int tm, tn, split, tiles_n;
};
// position of block `bid` of an `nb`-block grid when the grid is read XCD by XCD
MTB_DEV int xcd_order(int bid, int nb) { return (nb & 7) == 0 ? (bid & 7) * (nb >> 3) + (bid >> 3) : bid; }
// tile of the block at XCD-ordered position `bid` of one product
template <int BM, int BN>
MTB_DEV BlockTile tile_at(int M, int N, int bid) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int split = bid / (tiles_m * tiles_n);
  bid -= split * (tiles_m * tiles_n);
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int first_m = (bid / per_group) * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  return {first_m + (bid % per_group) % gsz, (bid % per_group) / gsz, split, tiles_n};
}
template <int BM, int BN>
MTB_DEV BlockTile block_tile(int M, int N) {
  return tile_at<BM, BN>(M, N, xcd_order(blockIdx.x, gridDim.x));
}

// Epilogue. lane holds C[m][n..n+3] with m = (lane & 31), n = 8q + 4(lane >> 5)
// inside each 32x32 fragment (register 4q + r -> column n + r). The tile goes
// through LDS CR rows at a time, reusing the operand buffers (SMEM_F floats;
// the caller has synchronised after the last operand read).
template <int BM, int BN, int WGM, int WGN, int SMEM_F, bool AKC, int EPI, bool RPRE = false>
MTB_DEV void gemm_epilogue(const f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32], void* smem,
                           const Epi& ep, int M, int N, int m0, int n0, const BlockTile& bt,
                           int wm, int wn, int lane, int tid) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  constexpr int CR = stage_rows(BM, WM, SMEM_F / BN, BM);
  static_assert(CR >= WM && BM % CR == 0 && CR * BN <= SMEM_F, "staging chunk");
  const Staged<BN> st{reinterpret_cast<float*>(smem)};
  // RPRE (plain stores with a residual, EPI_DGELU, EPI_DSWIGLU): a chunk's
  // row operand is requested in full before any of its stores -- chunk 0's
  // before the staging, chunk c + 1's right after chunk c's stores (vector
  // memory operations complete in issue order, so a load issued after a store
  // is waited for behind that store: one wait per chunk instead of one per
  // row item); EPI_DSWIGLU's two operands go half a chunk at a time (one wait
  // per half). For kernels whose accumulators live in AGPRs; in the
  // 2x4-wavefront kernel the extra registers spill.
  constexpr bool PRE = RPRE && (EPI == EPI_STORE || EPI == EPI_DGELU);
  RowOperand<BN, CR, NT> pre;
  auto load_pre = [&](int mc) {
    if constexpr (EPI == EPI_STORE)
      pre.load(ep.resid, ep.ldr, M, N, mc, n0, tid);
    else
      pre.load(ep.aux, ep.ldaux, M, N, mc, n0, tid);
  };
  const bool has_pre = PRE && (EPI == EPI_STORE ? ep.resid : ep.aux) != nullptr;
  if constexpr (PRE) {
    if (has_pre) load_pre(m0);
  }
  // EPI_DSWIGLU: half a chunk of gate/up pre-activations at a time
  constexpr bool PRE_SWI = RPRE && EPI == EPI_DSWIGLU;
  SwiRows<BN, CR, NT> spre;
  const bool has_swi = PRE_SWI && ep.aux != nullptr;
  if constexpr (PRE_SWI) {
    if (has_swi) spre.load(ep, M, N, m0, n0, tid, 0);
  }
#pragma unroll 1
  for (int c0 = 0; c0 < BM; c0 += CR) {
    if (c0 > 0) __syncthreads();
    if (wm * WM >= c0 && wm * WM < c0 + CR) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM - c0 + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = wn * WN + j * 32 + 8 * q + 4 * (lane >> 5);
            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                             acc[i][j][4 * q + 3]};
            st.put4(r, n, v);
          }
      }
    }
    __syncthreads();
    // the row items' LDS and global addresses are the same for every chunk;
    // hidden behind this copy of tid they are recomputed per chunk instead of
    // held (or spilled) across the loop
    int t = tid;
    asm volatile("" : "+v"(t));
    if constexpr (EPI == EPI_PARTIAL)
      epi_partial<BN, CR, NT>(reinterpret_cast<float*>(ep.ws) + (size_t)bt.split * M * N, st, M, N,
                              m0 + c0, n0, t);
    else if constexpr (EPI == EPI_XENT_STATS)
      epi_xent_stats<BN, CR, NT>(ep, st, M, N, m0 + c0, n0, bt.tn, bt.tiles_n, t);
    else if (has_pre)
      epi_rows_pre<PRE ? EPI : EPI_STORE, BN, CR, NT>(ep, st, M, N, m0 + c0, n0, t, pre);
    else if (has_swi)
      epi_rows_dswiglu_pre<BN, CR, NT>(ep, st, M, N, m0 + c0, n0, t, spre);
    else
      epi_rows<EPI, BN, CR, NT>(ep, st, M, N, m0 + c0, n0, t);
    if constexpr (PRE) {
      if (has_pre && c0 + CR < BM) load_pre(m0 + c0 + CR);
    }
    if constexpr (PRE_SWI) {
      if (has_swi && c0 + CR < BM) spre.load(ep, M, N, m0 + c0 + CR, n0, tid, 0);
    }
  }
}

// BM x BN block tile, WGM x WGN wavefronts (each WM x WN = FM x FN 32x32
// fragments), OCC = wavefronts per SIMD the register budget must allow
template <int BM, int BN, int WGM, int WGN, int OCC, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN, OCC) void gemm_bf16_kernel(int M, int N, int K,
                                                           const bf16_t* __restrict__ A, int lda,
                                                           const bf16_t* __restrict__ B, int ldb,
                                                           Epi ep, int ksplit) {
  constexpr int NT = 64 * WGM * WGN;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  // operand double buffers; reused by the epilogue for the staged fp32 tile
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * (BM + BN) * BK];
  auto sA = [&](int i) { return smem + i * (BM * BK); };
  auto sB = [&](int i) { return smem + 2 * BM * BK + i * (BN * BK); };
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  const BlockTile bt = block_tile<BM, BN>(M, N);
  const int kspan = K / ksplit, kbeg = bt.split * kspan;
  const int m0 = bt.tm * BM, n0 = bt.tn * BN;

  using LA = typename std::conditional<AKC, TileKc<BM, NT>, TileMnT<BM, NT>>::type;
  using LB = typename std::conditional<BKC, TileKc<BN, NT>, TileMnT<BN, NT>>::type;
  LA la;
  LB lb;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int KT = (kspan + BK - 1) / BK, kend = kbeg + kspan;
  la.load(A, lda, m0, M, kbeg, kend, tid);
  lb.load(B, ldb, n0, N, kbeg, kend, tid);
  la.store(sA(0), tid);
  lb.store(sB(0), tid);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      la.load(A, lda, m0, M, kbeg + (kt + 1) * BK, kend, tid);
      lb.load(B, ldb, n0, N, kbeg + (kt + 1) * BK, kend, tid);
    }
    const bf16_t* as = sA(cur);
    const bf16_t* bs = sB(cur);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      bf16x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        if constexpr (AKC)
          af[i] = *reinterpret_cast<const bf16x8*>(as + row * BK + ((c ^ swz(row)) << 3));
        else
          af[i] = frag_tr<BM>(as, wm * WM + i * 32, kk, lane);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WN + j * 32 + (lane & 31);
        if constexpr (BKC)
          bf[j] = *reinterpret_cast<const bf16x8*>(bs + row * BK + ((c ^ swz(row)) << 3));
        else
          bf[j] = frag_tr<BN>(bs, wn * WN + j * 32, kk, lane);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      la.store(sA(cur ^ 1), tid);
      lb.store(sB(cur ^ 1), tid);
    }
    __syncthreads();
  }

  gemm_epilogue<BM, BN, WGM, WGN, (BM + BN) * BK, AKC, EPI>(acc, smem, ep, M, N, m0, n0, bt, wm, wn,
                                                            lane, tid);
}

// Hand-scheduled tiles: 2 x WGN wavefronts, each with FM x FN 32x32
// accumulators, the k-loop one inline-assembly block of gemm_loop.inc
// (schedules and LDS layout: gen_gemm_loop.py). Shapes, all with 4 stages and
// one block per CU:
//   SH256:   256 x 256 on 4 wavefronts (2 x 2) of 128 x 128;
//   SH192:   256 x 192 on 4 wavefronts of 128 x 96 (1536-wide products: 256
//            tiles on 256 CUs instead of 192);
//   SH256W8: 256 x 256 on 8 wavefronts (2 x 4) of 128 x 64, two per SIMD, so
//            that one wavefront's MFMAs run while the other waits on its
//            copies, fragment reads or the barrier;
//   SH128:   128 x 128 on 4 wavefronts of 64 x 64, two blocks per CU (64 KB
//            of LDS each): for products whose larger tiles leave CUs idle,
//            one block's first copies and epilogue overlap the other's loop;
//   SH192W8: 256 x 192 on 8 wavefronts (4 x 2) of 64 x 96, k-contiguous
//            operands and contractions that are a multiple of 64 only (the
//            64-deep loop: its B tile's 24 copy blocks split over 8
//            wavefronts, the 32-deep tile's 12 do not).
// Needs each split's contraction to be a multiple of 32 and every operand
// byte offset below 2^32 (sched_ok).
constexpr int SBK = 32;
enum SchedShape { SH256 = 0, SH192 = 1, SH256W8 = 2, SH128 = 3, SH192W8 = 4 };
template <int SH>
struct Sched {
  static constexpr int WAVES = SH == SH256W8 || SH == SH192W8 ? 8 : 4;
  static constexpr int WGN = SH == SH192W8 ? 2 : WAVES / 2, WGM = WAVES / WGN;  // wavefront grid
  static constexpr int FM = SH == SH128 || SH == SH192W8 ? 2 : 4;
  static constexpr int FN = SH == SH256 ? 4 : SH == SH192 || SH == SH192W8 ? 3 : 2;
  static constexpr int BM = 32 * WGM * FM, BN = 32 * WGN * FN;
  static constexpr int STAGES = 4;
  static constexpr int SLOTS = STAGES;                 // loop body slots (gen_gemm_loop.py)
  static constexpr int PER_CU = SH == SH128 ? 2 : 1;
  static constexpr int QA = BM / 16 / WAVES, QB = BN / 16 / WAVES;  // copy blocks per wavefront and k-tile
  static constexpr uint32_t STAGE_BYTES = (BM + BN) * SBK * 2;
  static constexpr int SETS = (STAGES + 1) / 2;       // fragment base sets (stages 2i, 2i+1)
  static constexpr int SMEM = STAGES * (BM + BN) * SBK;  // bf16 elements of LDS
};

// the 256 x 256 shape every scheduled launch of that tile uses: two
// wavefronts per SIMD measured 4-7 % faster than one on the block's products
// with k-contiguous operands (fc1 forward 134 -> 129 us, fc1 dgrad 116 -> 110
// us) and the same on the weight gradients
constexpr int kShMain = SH256W8;

// The 32-deep loop: copies and fragment bases for the layout of
// gen_gemm_loop.py's Shape (4 stages), then its asm block.
template <int SH, bool AKC, bool BKC>
MTB_DEV void sched_loop32(f32x16 (&acc)[Sched<SH>::FM][Sched<SH>::FN], uint32_t lds, int M, int N,
                          const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb,
                          int kbeg, int kspan, int m0, int n0, int wave, int wm, int wn, int lane) {
  using G = Sched<SH>;
  constexpr int BM = G::BM, BN = G::BN, FM = G::FM, FN = G::FN;
  constexpr uint32_t B_OFF = BM * SBK * 2;  // operand B follows A inside a stage (bytes)
  // Copies: this wavefront's blocks Q wave + q (q < Q) of 1 KB per operand and
  // k-tile; lane l writes bytes [16 l, 16 l + 16) of its block.
  // k-contiguous: block = 16 rows x 64 bytes; row r's chunk c sits at c ^ ((r >> 2) & 3).
  // otherwise:    block = 1024 / (2 ROWS) k-rows of 2 ROWS bytes; k-row k's chunk c sits at
  //               c ^ ((k & 3) << 2).
  auto copy_off = [&](bool kc, int b, int row0, int rows, int ld, int ROWS) -> uint32_t {
    if (kc) {
      const int r = 16 * b + (lane >> 2), c = (lane & 3) ^ ((r >> 2) & 3);
      return ((uint32_t)min(row0 + r, rows - 1) * (uint32_t)ld + c * 8) * 2u;
    }
    const int cpr = ROWS / 8, kpb = 64 / cpr;   // chunks per k-row, k-rows per block
    const int k = kpb * b + lane / cpr, c = (lane % cpr) ^ ((k & 3) << 2);
    return ((uint32_t)k * (uint32_t)ld + (uint32_t)min(row0 + c * 8, rows - 8)) * 2u;
  };
  uint32_t voA[G::QA], voB[G::QB];
#pragma unroll
  for (int q = 0; q < G::QA; ++q) voA[q] = copy_off(AKC, G::QA * wave + q, m0, M, lda, BM);
#pragma unroll
  for (int q = 0; q < G::QB; ++q) voB[q] = copy_off(BKC, G::QB * wave + q, n0, N, ldb, BN);
  const uint64_t sbA = (uint64_t)(A + (AKC ? (size_t)kbeg : (size_t)kbeg * lda));
  const uint64_t sbB = (uint64_t)(B + (BKC ? (size_t)kbeg : (size_t)kbeg * ldb));
  const uint32_t ksA = AKC ? SBK * 2 : SBK * 2 * (uint32_t)lda;
  const uint32_t ksB = BKC ? SBK * 2 : SBK * 2 * (uint32_t)ldb;
  const uint32_t ldsA = __builtin_amdgcn_readfirstlane(lds + wave * G::QA * 1024);
  const uint32_t ldsB = __builtin_amdgcn_readfirstlane(lds + B_OFF + wave * G::QB * 1024);

  // Fragment base addresses; set i (stages 2i, 2i+1) 2 i STAGE_BYTES further,
  // so that every read offset fits the 16-bit immediate.
  // k-contiguous: f[2 set + kk] for step kk (fragment i is 2 KB further);
  // otherwise: f[F set + i] for fragment i (step kk is 32 ROWS bytes further).
  constexpr int NA = G::SETS * (AKC ? 2 : FM), NB = G::SETS * (BKC ? 2 : FN);
  auto frag_bases = [&](bool kc, int w, uint32_t off, int F, int ROWS, uint32_t* f) {
    if (kc) {
      const int r = w * 32 * F + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = 2 * kk + (lane >> 5);
        const uint32_t b0 = lds + off + r * 64 + ((c ^ ((r >> 2) & 3)) << 4);
#pragma unroll
        for (int st = 0; st < G::SETS; ++st) f[2 * st + kk] = b0 + st * 2 * G::STAGE_BYTES;
      }
    } else {
      const int g = lane >> 4, sl = lane & 15, k = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const int m = w * 32 * F + 32 * i + 16 * (g & 1) + 4 * (sl & 3);
        const uint32_t b0 = lds + off + (k * ROWS + ((m >> 3) ^ ((k & 3) << 2)) * 8 + (m & 7)) * 2;
#pragma unroll
        for (int st = 0; st < G::SETS; ++st) f[F * st + i] = b0 + st * 2 * G::STAGE_BYTES;
      }
    }
  };
  uint32_t fa[NA], fb[NB];
  frag_bases(AKC, wm, 0, FM, BM, fa);
  frag_bases(BKC, wn, B_OFF, FN, BN, fb);

  const int KT = kspan / SBK;
  const int first = (G::SLOTS - KT % G::SLOTS) % G::SLOTS;  // body slot of k-tile 0
  int rem = KT - 1, iters = (KT + first) / G::SLOTS;
  uint32_t ta, tb;
#define MTB_ACC_ROW(I)                                                                             \
  [c##I##0] "+a"(acc[I][0]), [c##I##1] "+a"(acc[I][1])
#define MTB_LOOP_COMMON                                                                            \
    [rem] "+s"(rem), [iters] "+s"(iters), [ta] "=&s"(ta), [tb] "=&s"(tb)                           \
  : [ldsA] "s"(ldsA), [ldsB] "s"(ldsB), [sbA] "s"(sbA), [sbB] "s"(sbB), [ksA] "s"(ksA),            \
    [ksB] "s"(ksB), [first] "s"(first)
  // The loop writes M0 (the LDS address of its copies) before every use; no
  // code around it keeps a value in M0, so its clobber is declared without
  // the compiler's warning about reserved registers.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (SH == SH256) {
#define MTB_LOOP_OPERANDS                                                                          \
  : [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c02] "+a"(acc[0][2]), [c03] "+a"(acc[0][3]),    \
    [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]), [c12] "+a"(acc[1][2]), [c13] "+a"(acc[1][3]),    \
    [c20] "+a"(acc[2][0]), [c21] "+a"(acc[2][1]), [c22] "+a"(acc[2][2]), [c23] "+a"(acc[2][3]),    \
    [c30] "+a"(acc[3][0]), [c31] "+a"(acc[3][1]), [c32] "+a"(acc[3][2]), [c33] "+a"(acc[3][3]),    \
    [voA0] "+v"(voA[0]), [voA1] "+v"(voA[1]), [voA2] "+v"(voA[2]), [voA3] "+v"(voA[3]),            \
    [voB0] "+v"(voB[0]), [voB1] "+v"(voB[1]), [voB2] "+v"(voB[2]), [voB3] "+v"(voB[3]),            \
    MTB_LOOP_COMMON,                                                                               \
    [fa0] "v"(fa[0]), [fa1] "v"(fa[1]), [fa2] "v"(fa[2]), [fa3] "v"(fa[3]),                        \
    [fa4] "v"(fa[NA > 4 ? 4 : 0]), [fa5] "v"(fa[NA > 5 ? 5 : 0]), [fa6] "v"(fa[NA > 6 ? 6 : 0]),   \
    [fa7] "v"(fa[NA > 7 ? 7 : 0]),                                                                 \
    [fb0] "v"(fb[0]), [fb1] "v"(fb[1]), [fb2] "v"(fb[2]), [fb3] "v"(fb[3]),                        \
    [fb4] "v"(fb[NB > 4 ? 4 : 0]), [fb5] "v"(fb[NB > 5 ? 5 : 0]), [fb6] "v"(fb[NB > 6 ? 6 : 0]),   \
    [fb7] "v"(fb[NB > 7 ? 7 : 0])                                                                  \
  : "memory", "m0", "scc"
    if constexpr (AKC && BKC)
      asm volatile(MTB_GEMM_LOOP_NT MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_NT);
    else if constexpr (AKC)
      asm volatile(MTB_GEMM_LOOP_NN MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_NN);
    else
      asm volatile(MTB_GEMM_LOOP_TN MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_TN);
#undef MTB_LOOP_OPERANDS
  } else if constexpr (SH == SH192) {
    static_assert(AKC && BKC, "the 256 x 192 tile is built for k-contiguous operands only");
    asm volatile(MTB_GEMM_LOOP_NT_192
                 : [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c02] "+a"(acc[0][2]),
                   [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]), [c12] "+a"(acc[1][2]),
                   [c20] "+a"(acc[2][0]), [c21] "+a"(acc[2][1]), [c22] "+a"(acc[2][2]),
                   [c30] "+a"(acc[3][0]), [c31] "+a"(acc[3][1]), [c32] "+a"(acc[3][2]),
                   [voA0] "+v"(voA[0]), [voA1] "+v"(voA[1]), [voA2] "+v"(voA[2]), [voA3] "+v"(voA[3]),
                   [voB0] "+v"(voB[0]), [voB1] "+v"(voB[1]), [voB2] "+v"(voB[2]),
                   MTB_LOOP_COMMON,
                   [fa0] "v"(fa[0]), [fa1] "v"(fa[1]), [fa2] "v"(fa[2]), [fa3] "v"(fa[3]),
                   [fb0] "v"(fb[0]), [fb1] "v"(fb[1]), [fb2] "v"(fb[2]), [fb3] "v"(fb[3])
                 : "memory", "m0", "scc", MTB_GEMM_LOOP_CLOBBERS_NT_192);
  } else if constexpr (SH == SH256W8) {
#define MTB_LOOP_OPERANDS                                                                          \
  : [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]),    \
    [c20] "+a"(acc[2][0]), [c21] "+a"(acc[2][1]), [c30] "+a"(acc[3][0]), [c31] "+a"(acc[3][1]),    \
    [voA0] "+v"(voA[0]), [voA1] "+v"(voA[1]), [voB0] "+v"(voB[0]), [voB1] "+v"(voB[1]),            \
    MTB_LOOP_COMMON,                                                                               \
    [fa0] "v"(fa[0]), [fa1] "v"(fa[1]), [fa2] "v"(fa[2]), [fa3] "v"(fa[3]),                        \
    [fa4] "v"(fa[NA > 4 ? 4 : 0]), [fa5] "v"(fa[NA > 5 ? 5 : 0]), [fa6] "v"(fa[NA > 6 ? 6 : 0]),   \
    [fa7] "v"(fa[NA > 7 ? 7 : 0]),                                                                 \
    [fb0] "v"(fb[0]), [fb1] "v"(fb[1]), [fb2] "v"(fb[2]), [fb3] "v"(fb[3])                         \
  : "memory", "m0", "scc"
    if constexpr (AKC && BKC)
      asm volatile(MTB_GEMM_LOOP_NT_W8 MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_NT_W8);
    else if constexpr (AKC)
      asm volatile(MTB_GEMM_LOOP_NN_W8 MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_NN_W8);
    else
      asm volatile(MTB_GEMM_LOOP_TN_W8 MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_TN_W8);
#undef MTB_LOOP_OPERANDS
  } else if constexpr (SH == SH128) {
#define MTB_LOOP_OPERANDS                                                                          \
  : [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]),    \
    [voA0] "+v"(voA[0]), [voA1] "+v"(voA[1]), [voB0] "+v"(voB[0]), [voB1] "+v"(voB[1]),            \
    MTB_LOOP_COMMON,                                                                               \
    [fa0] "v"(fa[0]), [fa1] "v"(fa[1]), [fa2] "v"(fa[2]), [fa3] "v"(fa[3]),                        \
    [fb0] "v"(fb[0]), [fb1] "v"(fb[1]), [fb2] "v"(fb[2]), [fb3] "v"(fb[3])                         \
  : "memory", "m0", "scc"
    if constexpr (AKC && BKC)
      asm volatile(MTB_GEMM_LOOP_NT_128 MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_NT_128);
    else if constexpr (AKC)
      asm volatile(MTB_GEMM_LOOP_NN_128 MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_NN_128);
    else
      asm volatile(MTB_GEMM_LOOP_TN_128 MTB_LOOP_OPERANDS, MTB_GEMM_LOOP_CLOBBERS_TN_128);
#undef MTB_LOOP_OPERANDS
  }
#pragma clang diagnostic pop
#undef MTB_LOOP_COMMON
#undef MTB_ACC_ROW
}

// The 64-deep loop of the 8-wavefront tile (contractions that are a multiple
// of 64): two stages of [A BM x 64 | B BN x 64] in the same LDS as four
// 32-deep ones, so that a k-contiguous operand's copies move whole 128-byte
// lines (8 rows x 128 bytes per instruction) and the L2 serves half the
// requests of the 32-deep loop's 64-byte ones; copies and fragment bases for
// gen_gemm_loop.py's Shape64, then its asm block.
template <int SH, bool AKC, bool BKC>
MTB_DEV void sched_loop64(f32x16 (&acc)[Sched<SH>::FM][Sched<SH>::FN], uint32_t lds, int M, int N,
                          const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb,
                          int kbeg, int kspan, int m0, int n0, int wave, int wm, int wn, int lane) {
  static_assert(SH == SH256W8 || SH == SH192W8, "the 64-deep loop is built for the 8-wavefront tiles");
  using G = Sched<SH>;
  constexpr int BM = G::BM, BN = G::BN, FM = G::FM, FN = G::FN;
  constexpr uint32_t ST = (BM + BN) * 128, B_OFF = BM * 128;   // stage and operand-B offsets (bytes)
  constexpr int QA = BM * 128 / 1024 / G::WAVES, QB = BN * 128 / 1024 / G::WAVES;
  // Copies: this wavefront's blocks Q wave + q (q < Q) of 1 KB per operand and
  // k-tile; lane l writes bytes [16 l, 16 l + 16) of its block.
  // k-contiguous: block = 8 rows x 128 bytes (whole cache lines); row r's
  //               chunk j sits at j ^ ((r >> 1) & 7).
  // otherwise:    block = 1024 / (2 ROWS) k-rows of 2 ROWS bytes; k-row k's chunk c sits at
  //               c ^ ((k & 3) << 2).
  auto copy_off = [&](bool kc, int b, int row0, int rows, int ld, int ROWS) -> uint32_t {
    if (kc) {
      const int r = 8 * b + (lane >> 3), j = (lane & 7) ^ ((r >> 1) & 7);
      return ((uint32_t)min(row0 + r, rows - 1) * (uint32_t)ld + j * 8) * 2u;
    }
    const int cpr = ROWS / 8, kpb = 64 / cpr;
    const int k = kpb * b + lane / cpr, c = (lane % cpr) ^ ((k & 3) << 2);
    return ((uint32_t)k * (uint32_t)ld + (uint32_t)min(row0 + c * 8, rows - 8)) * 2u;
  };
  uint32_t voA[QA], voB[QB];
#pragma unroll
  for (int q = 0; q < QA; ++q) voA[q] = copy_off(AKC, QA * wave + q, m0, M, lda, BM);
#pragma unroll
  for (int q = 0; q < QB; ++q) voB[q] = copy_off(BKC, QB * wave + q, n0, N, ldb, BN);
  const uint64_t sbA = (uint64_t)(A + (AKC ? (size_t)kbeg : (size_t)kbeg * lda));
  const uint64_t sbB = (uint64_t)(B + (BKC ? (size_t)kbeg : (size_t)kbeg * ldb));
  const uint32_t ksA = AKC ? 128u : 128u * (uint32_t)lda;
  const uint32_t ksB = BKC ? 128u : 128u * (uint32_t)ldb;
  const uint32_t ldsA = __builtin_amdgcn_readfirstlane(lds + wave * QA * 1024);
  const uint32_t ldsB = __builtin_amdgcn_readfirstlane(lds + B_OFF + wave * QB * 1024);

  // Fragment base addresses, one per stage and: step s (k-contiguous; its
  // fragment i is 32 rows = 4 KB further) or fragment i (otherwise; step s
  // is 16 k-rows further, a fragment's second half 4 k-rows).
  constexpr int NA = 2 * (AKC ? 4 : FM), NB = 2 * (BKC ? 4 : FN);
  auto frag_bases = [&](bool kc, int w, uint32_t off, int F, int ROWS, uint32_t* f) {
    if (kc) {
      const int r = w * 32 * F + (lane & 31);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = 2 * q + (lane >> 5);
          f[4 * st + q] = lds + off + st * ST + r * 128 + ((j ^ ((r >> 1) & 7)) << 4);
        }
    } else {
      const int g = lane >> 4, sl = lane & 15, k = 8 * (g >> 1) + (sl >> 2);
#pragma unroll
      for (int i = 0; i < F; ++i) {
        const int m = w * 32 * F + 32 * i + 16 * (g & 1) + 4 * (sl & 3);
        const uint32_t b0 = lds + off + (k * ROWS + ((m >> 3) ^ ((k & 3) << 2)) * 8 + (m & 7)) * 2;
#pragma unroll
        for (int st = 0; st < 2; ++st) f[F * st + i] = b0 + st * ST;
      }
    }
  };
  uint32_t fa[NA], fb[NB];
  frag_bases(AKC, wm, 0, FM, BM, fa);
  frag_bases(BKC, wn, B_OFF, FN, BN, fb);

  const int KT = kspan / 64;
  const int first = KT & 1;  // body slot of k-tile 0 (-KT mod 2)
  int rem = KT - 1, iters = (KT + first) / 2;
  uint32_t ta, tb;
  static_assert(AKC && BKC && NA == 8 && NB == 8, "the 64-deep loop is built for k-contiguous operands");
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
#define MTB_LOOP_COMMON                                                                            \
    [rem] "+s"(rem), [iters] "+s"(iters), [ta] "=&s"(ta), [tb] "=&s"(tb)                           \
  : [ldsA] "s"(ldsA), [ldsB] "s"(ldsB), [sbA] "s"(sbA), [sbB] "s"(sbB), [ksA] "s"(ksA),            \
    [ksB] "s"(ksB), [first] "s"(first),                                                            \
    [fa0] "v"(fa[0]), [fa1] "v"(fa[1]), [fa2] "v"(fa[2]), [fa3] "v"(fa[3]),                        \
    [fa4] "v"(fa[4]), [fa5] "v"(fa[5]), [fa6] "v"(fa[6]), [fa7] "v"(fa[7]),                        \
    [fb0] "v"(fb[0]), [fb1] "v"(fb[1]), [fb2] "v"(fb[2]), [fb3] "v"(fb[3]),                        \
    [fb4] "v"(fb[4]), [fb5] "v"(fb[5]), [fb6] "v"(fb[6]), [fb7] "v"(fb[7])                         \
  : "memory", "m0", "scc"
  if constexpr (SH == SH256W8)
    asm volatile(MTB_GEMM_LOOP64_NT_W8
                 : [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]),
                   [c20] "+a"(acc[2][0]), [c21] "+a"(acc[2][1]), [c30] "+a"(acc[3][0]), [c31] "+a"(acc[3][1]),
                   [voA0] "+v"(voA[0]), [voA1] "+v"(voA[1]), [voA2] "+v"(voA[2]), [voA3] "+v"(voA[3]),
                   [voB0] "+v"(voB[0]), [voB1] "+v"(voB[1]), [voB2] "+v"(voB[2]), [voB3] "+v"(voB[3]),
                   MTB_LOOP_COMMON, MTB_GEMM_LOOP_CLOBBERS64_NT_W8);
  else
    asm volatile(MTB_GEMM_LOOP64_NT_192W8
                 : [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c02] "+a"(acc[0][2]),
                   [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]), [c12] "+a"(acc[1][2]),
                   [voA0] "+v"(voA[0]), [voA1] "+v"(voA[1]), [voA2] "+v"(voA[2]), [voA3] "+v"(voA[3]),
                   [voB0] "+v"(voB[0]), [voB1] "+v"(voB[1]), [voB2] "+v"(voB[2]),
                   MTB_LOOP_COMMON, MTB_GEMM_LOOP_CLOBBERS64_NT_192W8);
#undef MTB_LOOP_COMMON
#pragma clang diagnostic pop
}

// One block's tile (bt) of the product: the k-loop and the epilogue. smem is
// the block's Sched<SH>::SMEM-element LDS array (1-KB aligned).
template <int SH, bool AKC, bool BKC, int EPI>
MTB_DEV void sched_tile(bf16_t* smem, int M, int N, int K, const bf16_t* __restrict__ A, int lda,
                        const bf16_t* __restrict__ B, int ldb, const Epi& ep, int ksplit,
                        const BlockTile& bt, bool prefetch_b = false) {
  using G = Sched<SH>;
  constexpr int BM = G::BM, BN = G::BN, FM = G::FM, FN = G::FN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / G::WGN, wn = wave % G::WGN;
  const int kspan = K / ksplit, kbeg = bt.split * kspan;
  const int m0 = bt.tm * BM, n0 = bt.tn * BN;
  const uint32_t lds = (uint32_t)(uintptr_t)smem;
  // B operand prefetch for a small B (at most 8 MB: a weight matrix that
  // many blocks share, such as the 4096 x 512 projection's) read by a deep
  // contraction or by two waves of blocks: the grid's
  // blocks each touch one slice of B's bytes (one 4-byte load per 128-byte
  // line, at most two per thread), so that the infinity cache holds B before
  // the k-loop's copies ask for it -- the step last read that weight long
  // ago, and when every block misses on the same cold lines each k-tile's
  // copy waits out the HBM latency (projection dgrad 60 -> 44 us). The loads
  // join the k-loop's first copy wait (vector memory operations complete in
  // issue order); their values are only kept alive. A large B (16 MB
  // weights, the weight gradients' activations) was slower with it.
  uint32_t pf0 = 0, pf1 = 0;
  if (prefetch_b) {
    constexpr int NT = 64 * G::WAVES;
    const size_t bytes = 2 * (BKC ? (size_t)(N - 1) * ldb + K : (size_t)(K - 1) * ldb + N);
    if (bytes <= ((size_t)8 << 20) && (K >= 2048 || gridDim.x >= 512)) {
      const size_t per = ((bytes + gridDim.x - 1) / gridDim.x + 127) & ~(size_t)127;
      const size_t lo = (size_t)blockIdx.x * per, hi = min(bytes, lo + per);
      const char* bb = reinterpret_cast<const char*>(B);
      const size_t o0 = lo + (size_t)tid * 128, o1 = o0 + (size_t)NT * 128;
      if (o0 + 4 <= hi) pf0 = *reinterpret_cast<const uint32_t*>(bb + o0);
      if (o1 + 4 <= hi) pf1 = *reinterpret_cast<const uint32_t*>(bb + o1);
    }
  }
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // the 64-deep loop where both operands are k-contiguous (both then copy
  // whole lines: fc1 forward 116.6 -> 109.0 us in a standalone run); with a
  // transposed operand, whose copies are whole lines in either loop, it was
  // 2-8 % slower (fc1 dgrad 119 -> 122 us, a weight gradient 130 -> 140 us)
  if constexpr (SH == SH192W8) {
    // launched only for contractions that are a multiple of 64 (launch_bf16)
    sched_loop64<SH, AKC, BKC>(acc, lds, M, N, A, lda, B, ldb, kbeg, kspan, m0, n0, wave, wm, wn, lane);
  } else {
    bool done = false;
    if constexpr (SH == SH256W8 && AKC && BKC) {
      if (kspan % 64 == 0) {
        sched_loop64<SH, AKC, BKC>(acc, lds, M, N, A, lda, B, ldb, kbeg, kspan, m0, n0, wave, wm, wn, lane);
        done = true;
      }
    }
    if (!done)
      sched_loop32<SH, AKC, BKC>(acc, lds, M, N, A, lda, B, ldb, kbeg, kspan, m0, n0, wave, wm, wn, lane);
  }
  asm volatile("" : : "v"(pf0), "v"(pf1));
  __syncthreads();
  gemm_epilogue<BM, BN, G::WGM, G::WGN, G::SMEM / 2, AKC, EPI, true>(acc, smem, ep, M, N, m0, n0, bt, wm,
                                                                     wn, lane, tid);
}

template <int SH, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(64 * Sched<SH>::WAVES, Sched<SH>::PER_CU) void gemm_bf16_sched_kernel(
    int M, int N, int K, const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb,
    Epi ep, int ksplit) {
  __shared__ __attribute__((aligned(1024))) bf16_t smem[Sched<SH>::SMEM];
  sched_tile<SH, AKC, BKC, EPI>(smem, M, N, K, A, lda, B, ldb, ep, ksplit,
                                block_tile<Sched<SH>::BM, Sched<SH>::BN>(M, N), true);
}

// One product of a grouped launch: its operands, split and block count.
struct SchedProb {
  int M, N, K;
  const bf16_t* A;
  int lda;
  const bf16_t* B;
  int ldb;
  int ksplit, blocks;
  Epi ep;
};

// Two independent products in one grid (same operand layouts and epilogue):
// the first p0.blocks blocks in XCD order take p0, the rest p1, so that a
// product whose tiles leave CUs idle shares the chip with another one.
template <int SH, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(64 * Sched<SH>::WAVES, Sched<SH>::PER_CU) void gemm_bf16_sched_pair_kernel(
    SchedProb p0, SchedProb p1) {
  __shared__ __attribute__((aligned(1024))) bf16_t smem[Sched<SH>::SMEM];
  const int r = xcd_order(blockIdx.x, gridDim.x);
  const bool second = r >= p0.blocks;  // uniform over the block
  const int M = second ? p1.M : p0.M, N = second ? p1.N : p0.N, K = second ? p1.K : p0.K;
  const bf16_t* A = second ? p1.A : p0.A;
  const bf16_t* B = second ? p1.B : p0.B;
  const int lda = second ? p1.lda : p0.lda, ldb = second ? p1.ldb : p0.ldb;
  const int ksplit = second ? p1.ksplit : p0.ksplit;
  const Epi ep = second ? p1.ep : p0.ep;
  sched_tile<SH, AKC, BKC, EPI>(smem, M, N, K, A, lda, B, ldb, ep, ksplit,
                                tile_at<Sched<SH>::BM, Sched<SH>::BN>(M, N, second ? r - p0.blocks : r));
}

// ---------------------------------------------------------------------------
// fp32 path: plain 64x64 register-blocked FMA GEMM (correctness-size problems)
// ---------------------------------------------------------------------------
template <bool AKC, bool BKC>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int M, int N, int K,
                                                       const float* __restrict__ A, int lda,
                                                       const float* __restrict__ B, int ldb,
                                                       Epi ep) {
  __shared__ float sA[16][68];
  __shared__ float sB[16][68];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      int row, kk;
      if (AKC) { row = e >> 4; kk = e & 15; } else { kk = e >> 6; row = e & 63; }
      const int gm = m0 + row, gk = k0 + kk;
      float va = 0.f;
      if (gm < M && gk < K) va = AKC ? A[(size_t)gm * lda + gk] : A[(size_t)gk * lda + gm];
      sA[kk][row] = va;
      if (BKC) { row = e >> 4; kk = e & 15; } else { kk = e >> 6; row = e & 63; }
      const int gn = n0 + row, gk2 = k0 + kk;
      float vb = 0.f;
      if (gn < N && gk2 < K) vb = BKC ? B[(size_t)gn * ldb + gk2] : B[(size_t)gk2 * ldb + gn];
      sB[kk][row] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { a[i] = sA[kk][ty * 4 + i]; b[i] = sB[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int n = n0 + tx * 4;
  if (n >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    epi4_f32(ep, m, n, N, v);
  }
}

template <int BM, int BN, int WGM, int WGN, int OCC, bool AKC, bool BKC, int EPI>
hipError_t launch_cfg(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                      const Epi& e, hipStream_t st, int ksplit = 1) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, OCC, AKC, BKC, EPI>), dim3(tiles * ksplit),
                     dim3(64 * WGM * WGN), 0, st, M, N, K, (const bf16_t*)A, lda,
                     (const bf16_t*)B, ldb, e, ksplit);
  return hipGetLastError();
}

constexpr int kCUs = 256;

// Fraction of the chip's block slots that `tiles` blocks keep busy over their
// waves (slots = kCUs * blocks per CU).
double fill(long tiles, int per_cu) {
  const long slots = (long)kCUs * per_cu, waves = (tiles + slots - 1) / slots;
  return (double)tiles / (double)(waves * slots);
}

enum Tile { T256x256, T256x192, T256x128, T128x128, TSCHED, TSCHED192 };
struct Plan {
  Tile tile;
  int splits;  // > 1: the contraction is split over that many blocks per tile
};

// Tile shape and contraction split per problem, the one decision both the
// launch and the workspace query use. Candidates (relative per-tile rates
// measured on MI355X over the block's GEMM shapes, times the fraction of the
// chip their tile count fills): the scheduled 256x256 kernel (8 wavefronts,
// gen_gemm_loop.py) when the contraction is a multiple of 32 and at least 1024
// deep, 1.2-1.5x the 2x4-wavefront 256x256 kernel; 256x192 (4x2 wavefronts)
// when N splits into 192-wide tiles (plain store); 128x128 (2x2, two blocks
// per CU). Weight gradients (both operands transposed in LDS) take the
// scheduled kernel with the contraction split until the blocks fill 3/4 of
// the chip; without it, 256x128 (4x2) when it fills the chip, else 128x128 (at
// two blocks per CU those beat a partly filled 256x128 grid: 158 vs 175 us for
// the 1536 x 4096 x 8192 QKV weight gradient). Tiles for 6 wavefronts fill the
// chip better at N = 1536 but leave two of a CU's four SIMDs with twice the
// work: measured slower.
//
// Split contraction (needs a workspace, `split_ok`; plain stores only): a
// deep product whose tiles leave at least half of the chip's block slots idle
// gets its contraction split into 2, 4 or 8 parts at least 1024 deep --
// token-major products on 128x128 tiles up to both blocks per CU -- and the
// fp32 partial tiles are summed in a fixed order by a second pass that also
// runs the epilogue. Each extra split costs 8 bytes per output element of
// partial-tile traffic. (At the seq-512 share, where every GEMM is 4096 x
// <=1024 x <=4096, splitting every product down to 512-deep parts made the
// step slower, 0.356 -> 0.401 ms: a block's fixed costs, not its k-loop,
// dominate there; only the gradients that would leave at least half of the
// chip idle go below 1024, see small_ok.)
Plan plan(int M, int N, int K, bool a_kc, bool b_kc, int kind, bool split_ok) {
  auto tl = [&](int bm, int bn) { return (long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  auto depth_ok = [&](int s) { return K % (s * BK) == 0 && K / s >= 1024; };
  // parts down to 512 deep for weight and data gradients whose blocks would
  // otherwise leave at least half of the chip's block slots idle (the
  // seq-512 share's 4096-token products: its four weight gradients and the
  // projection dgrad, step 0.354 -> 0.334 ms); forward products keep 1024
  // (the QKV forward's extra pass for its transposed copy cost more than the
  // split gained)
  auto small_ok = [&](int s) { return K % (s * BK) == 0 && K / s >= 512; };
  auto sched_depth = [&](int s) { return K % (s * SBK) == 0 && K / s >= 1024; };
  const long t256 = tl(256, 256);
  if (!a_kc && !b_kc) {
    if (K % SBK == 0) {
      int s = 1;
      if (split_ok && kind == EPI_STORE)
        while (s < 8 && t256 * s * 4 < 3L * kCUs && sched_depth(2 * s)) s *= 2;
      if (t256 * s * 2 >= kCUs) return {TSCHED, s};
    }
    const long t2 = tl(256, 128);
    if (split_ok && kind == EPI_STORE && t2 <= kCUs / 2 && K % BK == 0) {
      int s = 1;
      while (s < 8 && t2 * s * 4 < 3L * kCUs && (depth_ok(2 * s) || (t2 * s * 2 <= kCUs && small_ok(2 * s))))
        s *= 2;
      if (s > 1) return {T256x128, s};
    }
    if (K >= 1024 && t2 >= kCUs) return {T256x128, 1};
    return {T128x128, 1};
  }
  const long t128 = tl(128, 128);
  // token-major plain stores whose 256 x 256 tiles leave at least half of the
  // chip idle and whose contraction is deep (the 8192 x 512 x 4096 projection
  // data gradient: 64 tiles): the scheduled kernel on the contraction split
  // 2-4 ways into parts at least 1024 deep, then one pass that sums the
  // partial tiles and runs the epilogue
  // (not where the 256 x 256 tiles fill at most a quarter of the chip and
  // the scheduled 128 x 128 tiles alone give every CU a block: the 8192 x
  // 512 x 4096 projection dgrad, split 4 ways 49 + 13 -> 59 us; the 8192 x
  // 768 x 4096 QKV forward of the seq-4096 share stays split two ways, 63 +
  // 12 against 78 us)
  const bool fill128 = K % SBK == 0 && t128 >= kCUs && 4 * t256 <= kCUs;
  if (split_ok && a_kc && kind == EPI_STORE && 2 * t256 <= kCUs && K % SBK == 0 && !fill128) {
    int s = 1;
    while (s < 4 && t256 * s * 2 <= kCUs && sched_depth(2 * s)) s *= 2;
    // the 8-wavefront 256 x 192 tile where its split blocks fill more of the
    // chip (the seq-4096 share's 8192 x 768 x 4096 QKV forward: 96 tiles x 2
    // = 192 blocks -> 128 x 2 = 256; 67.0 -> 62.2 us standalone)
    if (b_kc && N % 192 == 0) {
      const long t192 = tl(256, 192);
      int s2 = 1;
      while (s2 < 4 && t192 * s2 * 2 <= kCUs && K % (2 * s2 * 64) == 0 && K / (2 * s2) >= 1024) s2 *= 2;
      if (s2 > 1 && t192 * s2 > t256 * s) return {TSCHED192, s2};
    }
    if (s > 1) return {TSCHED, s};
  }
  if (split_ok && a_kc && kind == EPI_STORE && t128 <= kCUs && t256 < kCUs && K % BK == 0 && !fill128) {
    int s = 1;
    while (s < 4 && t128 * s < 2L * kCUs && (depth_ok(2 * s) || (!b_kc && t128 * s < kCUs && small_ok(2 * s))))
      s *= 2;
    if (s > 1) return {T128x128, s};
  }
  // 128 x 128 tiles: the scheduled kernel (two blocks per CU) where the
  // contraction is a multiple of 32, else the 2x2-wavefront kernel. Where
  // both tiles fill the chip, the 256 x 256 one is faster (8192 x 4096 x 768:
  // 76 against 87 us); where the larger tiles leave CUs idle, the scheduled
  // 128 x 128 one wins (the seq-512 share's 4096-token products: 17.7 -> 13.2
  // us, 26.4 -> 19.9 us with the GELU' epilogue, its QKV forward 24.6 us on
  // 64 tiles of 256 x 192 -> 192 tiles of 128 x 128)
  const double f128 = (K % SBK == 0 ? 0.95 : 0.85) * fill(t128, 2);
  // the scheduled kernel from 512-deep contractions: on the 8-wavefront tile
  // it is the faster one there too (8192 x 4096 x 768 with a transposed
  // weight: 71 -> 55 us; 8192 x 4096 x 512, k-contiguous: 53 -> 43 us)
  const bool sk = K % SBK == 0 && K >= 512;
  if (K >= 512) {
    const double f256 = (sk ? 1.3 : 1.0) * fill(t256, 1);
    // 256 x 192 tiles: plain stores (the 2x4-wavefront kernel) or any epilogue (the scheduled one)
    const double f192 = (a_kc && b_kc && N % 192 == 0 && (sk || kind == EPI_STORE))
                            ? (sk ? 1.3 : 0.95) * fill(tl(256, 192), 1) : 0.0;
    if (f192 > f256 && f192 > f128) {
      // the scheduled 256 x 192 tile where it fills more of the chip than the 256 x 256 one
      // (the 8192 x 1536 QKV forward: 256 tiles instead of 192)
      if (sk) return {TSCHED192, 1};
      return {T256x192, 1};
    }
    if (f256 >= f128) return {sk ? TSCHED : T256x256, 1};
  }
  return {T128x128, 1};
}

// The scheduled 256 x 256 kernel takes a problem when each split's
// contraction is a multiple of 32 and every byte offset into an operand fits
// in 32 bits.
bool sched_ok(int M, int N, int K, bool a_kc, int lda, bool b_kc, int ldb, int splits) {
  if (K % splits != 0 || (K / splits) % SBK != 0) return false;
  auto fits = [&](bool kc, int rows, int ld) {
    const size_t last = kc ? (size_t)(rows - 1) * ld + K : (size_t)(K - 1) * ld + rows;
    return last * 2 < (size_t(1) << 32);
  };
  return M >= 8 && N >= 8 && fits(a_kc, M, lda) && fits(b_kc, N, ldb);
}

template <int SH, bool AKC, bool BKC, int EPI>
hipError_t launch_sched(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                        const Epi& e, hipStream_t st, int ksplit = 1) {
  constexpr int BM = Sched<SH>::BM, BN = Sched<SH>::BN;
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_bf16_sched_kernel<SH, AKC, BKC, EPI>), dim3(tiles * ksplit),
                     dim3(64 * Sched<SH>::WAVES), 0, st,
                     M, N, K, (const bf16_t*)A, lda, (const bf16_t*)B, ldb, e, ksplit);
  return hipGetLastError();
}

// Two weight gradients (both operands [K][rows], plain stores) in one grid of
// the scheduled kernel, in one of two forms:
//  - split: both contractions split 2, 4 or 8 ways, or p0 keeps the split
//    plan() gives it alone (its blocks leaving CUs idle) and p1 takes the
//    smallest split of at least two whose parts are no deeper than p0's; both
//    write fp32 partial tiles (p0's at ws, p1's after them) that the split
//    reduction sums;
//  - whole: neither is split, both products' tiles filling the chip together,
//    stored directly.
// A form is used when its blocks fill at least three quarters of the chip
// without exceeding it and a simple cost model puts it below the two launches
// one after the other: per wave of blocks, the k-tiles of one block plus 32
// k-tiles of fixed (prologue and epilogue) cost, and 16 k-tiles per split
// reduction pass.
struct PairPlan {
  bool ok = false;
  bool small = false;  // 128 x 128 tiles (two blocks per CU) instead of 256 x 256
  int s0 = 1, s1 = 1;
  size_t ws1 = 0;  // split form: byte offset of p1's partial tiles in the workspace
};
PairPlan pair_plan(int M0, int N0, int K0, int lda0, int ldb0, int M1, int N1, int K1, int lda1,
                   int ldb1) {
  PairPlan best;
  if (M0 <= 0 || N0 <= 0 || K0 <= 0 || M1 <= 0 || N1 <= 0 || K1 <= 0) return best;
  auto tiles = [](int m, int n, int bm, int bn) { return (long)((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  auto waves = [](long blocks, int per_cu) {
    return (blocks + (long)kCUs * per_cu - 1) / ((long)kCUs * per_cu);
  };
  // one product alone, on the tiles plan() gives it (k-tiles counted 32 deep whatever the kernel)
  auto alone = [&](const Plan& pl, int M, int N, int K) {
    const int bm = pl.tile == T128x128 ? 128 : 256;
    const int bn = pl.tile == T256x256 || pl.tile == TSCHED ? 256 : pl.tile == T256x192 || pl.tile == TSCHED192 ? 192 : 128;
    const int per = pl.tile == T128x128 ? 2 : 1;
    return waves(tiles(M, N, bm, bn) * pl.splits, per) * (K / pl.splits / SBK + 32) + (pl.splits > 1 ? 16 : 0);
  };
  const Plan a = plan(M0, N0, K0, false, false, EPI_STORE, true);
  const Plan b = plan(M1, N1, K1, false, false, EPI_STORE, true);
  long best_cost = alone(a, M0, N0, K0) + alone(b, M1, N1, K1);
  const long t0 = tiles(M0, N0, 256, 256), t1 = tiles(M1, N1, 256, 256);
  auto consider = [&](int s0, int s1) {
    if (K0 % (s0 * SBK) != 0 || K1 % (s1 * SBK) != 0 || K0 / s0 < 1024 || K1 / s1 < 1024) return;
    // a pair is there to fill the chip: at most a quarter of its CUs idle
    if (t0 * s0 + t1 * s1 > kCUs || 4 * (t0 * s0 + t1 * s1) < 3L * kCUs) return;
    if (!sched_ok(M0, N0, K0, false, lda0, false, ldb0, s0) || !sched_ok(M1, N1, K1, false, lda1, false, ldb1, s1))
      return;
    const long c = std::max(K0 / s0, K1 / s1) / SBK + 32 + (s0 > 1 ? 32 : 0);
    if (c >= best_cost) return;
    best_cost = c;
    best.ok = true;
    best.s0 = s0;
    best.s1 = s1;
    best.ws1 = s0 > 1 ? ((size_t)s0 * M0 * N0 * 4 + 255) & ~(size_t)255 : 0;
  };
  consider(1, 1);
  for (int sp = 2; sp <= 8; sp *= 2) consider(sp, sp);
  if (a.tile == TSCHED && a.splits >= 2) {
    int s1 = 2;
    while (s1 < 8 && K1 / s1 > K0 / a.splits) s1 *= 2;
    consider(a.splits, s1);
  }
  // Products too small for the scheduled 256 x 256 tiles, alone or paired
  // (the seq-512 share's 1024-wide weight gradients): the 128 x 128
  // scheduled tiles, two blocks per CU, both contractions split the same way
  // into parts at least 512 deep, with at least one block for every CU and at
  // most two. In the cost units above a 128 x 128 k-tile counts 1/3 of a 256
  // x 256 one (a quarter of its work at a lower rate), per block a CU holds.
  // Products that run on the 256 x 256 tiles alone stay there (the seq-4096
  // share's QKV and projection weight gradients: 13 us faster alone).
  if (!best.ok && a.tile != TSCHED && b.tile != TSCHED) {
    const long u0 = tiles(M0, N0, 128, 128), u1 = tiles(M1, N1, 128, 128);
    for (int sp = 1; sp <= 8; sp *= 2) {
      if (K0 % (sp * SBK) != 0 || K1 % (sp * SBK) != 0 || K0 / sp < 512 || K1 / sp < 512) continue;
      const long blocks = (u0 + u1) * sp;
      if (blocks < kCUs || blocks > 2L * kCUs) continue;
      if (!sched_ok(M0, N0, K0, false, lda0, false, ldb0, sp) || !sched_ok(M1, N1, K1, false, lda1, false, ldb1, sp))
        continue;
      const long per_cu = (blocks + kCUs - 1) / kCUs;
      const long c = std::max(K0, K1) / sp / SBK * per_cu / 3 + 16 + (sp > 1 ? 16 : 0);
      if (c >= best_cost) continue;
      best_cost = c;
      best.ok = best.small = true;
      best.s0 = best.s1 = sp;
      best.ws1 = sp > 1 ? ((size_t)sp * M0 * N0 * 4 + 255) & ~(size_t)255 : 0;
    }
  }
  return best;
}

// Column split of a forward product with an activation epilogue whose 256 x
// 256 tiles leave the last wave of blocks part-empty: the first n1 columns
// (a multiple of 256) on 256 x 256 tiles and the rest on 256 x 192 tiles,
// each part in whole waves, the 192-wide one three quarters as long (the
// seq-4096 share's SwiGLU fc1 forward, 8192 x 3584: 448 tiles in two waves,
// the second three quarters full -> 256 + 256 tiles). Returns n1, or 0 for
// no split.
int col_split_192(int M, int N, int K) {
  if (K % 64 != 0) return 0;
  const long rows = (M + 255) / 256;
  auto waves = [](long t) { return (t + kCUs - 1) / kCUs; };
  double best_c = (double)waves(rows * ((N + 255) / 256)) - 0.125;   // a gain of an eighth of a wave at least
  int best = 0;
  for (int n2 = 192; n2 < N; n2 += 192) {
    const int n1 = N - n2;
    if (n1 % 256 != 0) continue;
    const double c = (double)waves(rows * (n1 / 256)) + 0.75 * (double)waves(rows * (n2 / 192));
    if (c < best_c) {
      best_c = c;
      best = n1;
    }
  }
  return best;
}

template <bool AKC, bool BKC, int EPI>
hipError_t launch_bf16(int M, int N, int K, const void* A, int lda, const void* B, int ldb,
                       const Epi& e, hipStream_t st) {
  if constexpr (AKC && BKC && (EPI == EPI_SWIGLU || EPI == EPI_GELU)) {
    const int n1 = col_split_192(M, N, K);
    if (n1 > 0 && sched_ok(M, n1, K, AKC, lda, BKC, ldb, 1) && sched_ok(M, N - n1, K, AKC, lda, BKC, ldb, 1)) {
      const hipError_t r = launch_sched<kShMain, AKC, BKC, EPI>(M, n1, K, A, lda, B, ldb, e, st);
      if (r != hipSuccess) return r;
      // the second part's columns: SwiGLU's activation output holds half as
      // many (gate/up pairs of 16-column blocks; n1 is a multiple of 32)
      Epi e2 = e;
      e2.out = static_cast<bf16_t*>(e.out) + n1;
      e2.out2 = static_cast<bf16_t*>(e.out2) + (EPI == EPI_SWIGLU ? n1 / 2 : n1);
      if (e.bias) e2.bias = static_cast<const bf16_t*>(e.bias) + n1;
      return launch_sched<SH192W8, AKC, BKC, EPI>(M, N - n1, K, A, lda,
                                                  static_cast<const bf16_t*>(B) + (size_t)n1 * ldb, ldb, e2, st);
    }
  }
  const Plan pl = plan(M, N, K, AKC, BKC, EPI, e.ws != nullptr);
  if (pl.tile == TSCHED192) {
    if constexpr (AKC && BKC && EPI == EPI_STORE) {
      if (pl.splits > 1) {   // partial tiles (contraction parts multiples of 64), then the split epilogue pass
        if (!sched_ok(M, N, K, AKC, lda, BKC, ldb, pl.splits)) return hipErrorInvalidValue;
        const hipError_t r = launch_sched<SH192W8, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st, pl.splits);
        if (r != hipSuccess) return r;
        const unsigned tiles = (unsigned)(((M + 63) / 64) * ((N + 127) / 128));
        hipLaunchKernelGGL((splitk_epi_kernel<64, 128, 256, EPI>), dim3(tiles), dim3(256), 0, st, M, N,
                           pl.splits, (const float*)e.ws, e);
        return hipGetLastError();
      }
    }
    if constexpr (AKC && BKC) {
      if (sched_ok(M, N, K, AKC, lda, BKC, ldb, 1))
        return K % 64 == 0 ? launch_sched<SH192W8, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st)
                           : launch_sched<SH192, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
      if constexpr (EPI == EPI_STORE) return launch_cfg<256, 192, 4, 2, 1, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
    }
    return launch_cfg<256, 256, 2, 4, 1, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
  }
  if (pl.tile == TSCHED) {
    // operands past the 32-bit offsets: the 2x4-wavefront kernel on the same tiles
    const bool ok = sched_ok(M, N, K, AKC, lda, BKC, ldb, pl.splits);
    if constexpr (!AKC && !BKC && EPI == EPI_STORE) {
      if (pl.splits > 1) {
        const hipError_t r =
            ok ? launch_sched<kShMain, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st, pl.splits)
               : launch_cfg<256, 256, 2, 4, 1, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st,
                                                                       pl.splits);
        if (r != hipSuccess) return r;
        const size_t n8 = (size_t)M * N / 8;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           M, N, pl.splits, (const float*)e.ws, (bf16_t*)e.out, e.ldo);
        return hipGetLastError();
      }
    }
    if (pl.splits > 1) {
      // token-major plain stores: partial tiles, then the split epilogue pass
      if constexpr (AKC && EPI == EPI_STORE) {
        const hipError_t r =
            ok ? launch_sched<kShMain, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st, pl.splits)
               : launch_cfg<256, 256, 2, 4, 1, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st,
                                                                       pl.splits);
        if (r != hipSuccess) return r;
        const unsigned tiles = (unsigned)(((M + 63) / 64) * ((N + 127) / 128));
        hipLaunchKernelGGL((splitk_epi_kernel<64, 128, 256, EPI>), dim3(tiles), dim3(256), 0, st, M, N,
                           pl.splits, (const float*)e.ws, e);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
    return ok ? launch_sched<kShMain, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st)
              : launch_cfg<256, 256, 2, 4, 1, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
  }
  if (pl.splits > 1) {
    hipError_t r;
    if constexpr (!AKC && !BKC) {
      if (pl.tile == T256x128)
        r = launch_cfg<256, 128, 4, 2, 1, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st, pl.splits);
      else
        r = launch_cfg<128, 128, 2, 2, 2, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st, pl.splits);
      if (r != hipSuccess) return r;
      const size_t n8 = (size_t)M * N / 8;
      hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                         M, N, pl.splits, (const float*)e.ws, (bf16_t*)e.out, e.ldo);
    } else {
      r = (K / pl.splits) % SBK == 0 && sched_ok(M, N, K, AKC, lda, BKC, ldb, pl.splits)
              ? launch_sched<SH128, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st, pl.splits)
              : launch_cfg<128, 128, 2, 2, 2, AKC, BKC, EPI_PARTIAL>(M, N, K, A, lda, B, ldb, e, st,
                                                                      pl.splits);
      if (r != hipSuccess) return r;
      // 64-row pieces: twice the workgroups of the GEMM's tiles, two per CU, so
      // more of the partial-tile loads are in flight (15.0 -> 11.5 us for the
      // 8192 x 512 projection dgrad)
      const unsigned tiles = (unsigned)(((M + 63) / 64) * ((N + 127) / 128));
      hipLaunchKernelGGL((splitk_epi_kernel<64, 128, 256, EPI>), dim3(tiles), dim3(256), 0, st, M, N,
                         pl.splits, (const float*)e.ws, e);
    }
    return hipGetLastError();
  }
  if constexpr (!AKC && !BKC) {
    if (pl.tile == T256x128)
      return launch_cfg<256, 128, 4, 2, 1, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
  } else {
    if constexpr (AKC && BKC && EPI == EPI_STORE)
      if (pl.tile == T256x192)
        return launch_cfg<256, 192, 4, 2, 1, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
    if (pl.tile == T256x256)
      return launch_cfg<256, 256, 2, 4, 1, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
  }
  if (K % SBK == 0 && sched_ok(M, N, K, AKC, lda, BKC, ldb, 1))
    return launch_sched<SH128, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
  return launch_cfg<128, 128, 2, 2, 2, AKC, BKC, EPI>(M, N, K, A, lda, B, ldb, e, st);
}

}  // namespace

int gemm_tile_n(int M, int N, int K, bool a_kc, bool b_kc, int kind) {
  switch (plan(M, N, K, a_kc, b_kc, kind, false).tile) {
    case T256x256:
    case TSCHED: return 256;
    case T256x192:
    case TSCHED192: return 192;
    default: return 128;
  }
}

size_t gemm_ws_bytes(int dtype, int M, int N, int K, bool a_kc, bool b_kc, int kind) {
  if (dtype == 0 || M <= 0 || N <= 0 || K <= 0) return 0;
  const Plan pl = plan(M, N, K, a_kc, b_kc, kind, true);
  return pl.splits > 1 ? (size_t)pl.splits * M * N * 4 : 0;
}

size_t gemm_wgrad_pair_ws_bytes(int dtype, const GemmProb& p0, const GemmProb& p1) {
  if (dtype == 0) return 0;
  const PairPlan pp = pair_plan(p0.M, p0.N, p0.K, p0.lda, p0.ldb, p1.M, p1.N, p1.K, p1.lda, p1.ldb);
  if (pp.ok) return pp.s0 > 1 ? pp.ws1 + (size_t)pp.s1 * p1.M * p1.N * 4 : 0;
  return std::max(gemm_ws_bytes(dtype, p0.M, p0.N, p0.K, false, false, EPI_STORE),
                  gemm_ws_bytes(dtype, p1.M, p1.N, p1.K, false, false, EPI_STORE));
}

hipError_t gemm_wgrad_pair(int dtype, const GemmProb& p0, const GemmProb& p1, void* ws, hipStream_t st) {
  const PairPlan pp = dtype == 0 || ws == nullptr
                          ? PairPlan()
                          : pair_plan(p0.M, p0.N, p0.K, p0.lda, p0.ldb, p1.M, p1.N, p1.K, p1.lda, p1.ldb);
  if (!pp.ok) {
    for (const GemmProb* q : {&p0, &p1}) {
      Epi e = q->e;
      e.ws = ws;
      const hipError_t r = gemm(dtype, q->M, q->N, q->K, q->A, q->lda, false, q->B, q->ldb, false, e, st);
      if (r != hipSuccess) return r;
    }
    return hipSuccess;
  }
  SchedProb q[2];
  const GemmProb* src[2] = {&p0, &p1};
  const int splits[2] = {pp.s0, pp.s1};
  void* wsp[2] = {ws, (char*)ws + pp.ws1};
  for (int i = 0; i < 2; ++i) {
    const GemmProb& g = *src[i];
    q[i].M = g.M; q[i].N = g.N; q[i].K = g.K;
    q[i].A = (const bf16_t*)g.A; q[i].lda = g.lda;
    q[i].B = (const bf16_t*)g.B; q[i].ldb = g.ldb;
    q[i].ksplit = splits[i];
    const int tm = pp.small ? 128 : 256;
    q[i].blocks = ((g.M + tm - 1) / tm) * ((g.N + tm - 1) / tm) * splits[i];
    q[i].ep = Epi();
    if (pp.s0 > 1) {
      q[i].ep.ws = wsp[i];
    } else {
      q[i].ep.out = g.e.out;
      q[i].ep.ldo = g.e.ldo;
    }
  }
  const dim3 grid((unsigned)(q[0].blocks + q[1].blocks));
  const dim3 block(64 * (pp.small ? Sched<SH128>::WAVES : Sched<kShMain>::WAVES));
  if (pp.s0 == 1) {
    if (pp.small)
      hipLaunchKernelGGL((gemm_bf16_sched_pair_kernel<SH128, false, false, EPI_STORE>), grid, block, 0, st,
                         q[0], q[1]);
    else
      hipLaunchKernelGGL((gemm_bf16_sched_pair_kernel<kShMain, false, false, EPI_STORE>), grid, block, 0, st,
                         q[0], q[1]);
    return hipGetLastError();
  }
  if (pp.small)
    hipLaunchKernelGGL((gemm_bf16_sched_pair_kernel<SH128, false, false, EPI_PARTIAL>), grid, block, 0, st,
                       q[0], q[1]);
  else
    hipLaunchKernelGGL((gemm_bf16_sched_pair_kernel<kShMain, false, false, EPI_PARTIAL>), grid, block, 0, st,
                       q[0], q[1]);
  hipError_t r = hipGetLastError();
  if (r != hipSuccess) return r;
  SplitSum sum[2];
  unsigned nblk[2];
  for (int i = 0; i < 2; ++i) {
    const GemmProb& g = *src[i];
    sum[i] = {g.M, g.N, splits[i], (const float*)wsp[i], (bf16_t*)g.e.out, g.e.ldo};
    nblk[i] = (unsigned)(((size_t)g.M * g.N / 8 + 255) / 256);
  }
  hipLaunchKernelGGL(splitk_reduce_pair_kernel, dim3(nblk[0] + nblk[1]), dim3(256), 0, st, sum[0], sum[1],
                     (int)nblk[0]);
  return hipGetLastError();
}

hipError_t gemm(int dtype, int M, int N, int K, const void* A, int lda, bool a_kc, const void* B,
                int ldb, bool b_kc, const Epi& e, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == 0) {
    if (e.kind != EPI_STORE) return hipErrorInvalidValue;
    dim3 grid((N + 63) / 64, (M + 63) / 64);
#define MTB_F32G(AK, BKc)                                                                   \
  hipLaunchKernelGGL((gemm_f32_kernel<AK, BKc>), grid, dim3(256), 0, st, M, N, K,          \
                     (const float*)A, lda, (const float*)B, ldb, e)
    if (a_kc && b_kc) MTB_F32G(true, true);
    else if (a_kc) MTB_F32G(true, false);
    else if (b_kc) MTB_F32G(false, true);
    else MTB_F32G(false, false);
#undef MTB_F32G
    return hipGetLastError();
  }
  // bf16: K % 8 == 0 (a partial last k-tile is zero-filled), M % 8 == 0, N % 8 == 0 (checked by
  // the caller)
  if (a_kc && b_kc) {
    switch (e.kind) {
      case EPI_STORE: return launch_bf16<true, true, EPI_STORE>(M, N, K, A, lda, B, ldb, e, st);
      case EPI_GELU: return launch_bf16<true, true, EPI_GELU>(M, N, K, A, lda, B, ldb, e, st);
      case EPI_SWIGLU: return launch_bf16<true, true, EPI_SWIGLU>(M, N, K, A, lda, B, ldb, e, st);
      case EPI_XENT_STATS:
        return launch_bf16<true, true, EPI_XENT_STATS>(M, N, K, A, lda, B, ldb, e, st);
      case EPI_XENT_GRAD:
        return launch_bf16<true, true, EPI_XENT_GRAD>(M, N, K, A, lda, B, ldb, e, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (a_kc && !b_kc) {
    switch (e.kind) {
      case EPI_STORE: return launch_bf16<true, false, EPI_STORE>(M, N, K, A, lda, B, ldb, e, st);
      case EPI_DGELU: return launch_bf16<true, false, EPI_DGELU>(M, N, K, A, lda, B, ldb, e, st);
      case EPI_DSWIGLU: return launch_bf16<true, false, EPI_DSWIGLU>(M, N, K, A, lda, B, ldb, e, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (!a_kc && !b_kc && e.kind == EPI_STORE)
    return launch_bf16<false, false, EPI_STORE>(M, N, K, A, lda, B, ldb, e, st);
  return hipErrorInvalidValue;
}

}  // namespace mtb
