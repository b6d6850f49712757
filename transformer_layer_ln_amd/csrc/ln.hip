// LayerNorm forward/backward and the small elementwise / column-reduction
// kernels of the block. All are HBM-bound: one 64-lane wavefront owns one
// row, holds it in registers (16-byte vector loads, coalesced across lanes)
// and reduces with wavefront butterflies.
//
// LayerNorm: [Lab06] sec. 2 steps (2) and (5) -- F.layer_norm over the hidden
// dimension: per-token mean and biased variance, (x - mean) / sqrt(var + eps),
// optional gain/shift.
#include <algorithm>

#include "common.h"
#include "drop.h"
#include "kernels.h"

namespace mtb {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts, one row each

// 8 elements of a stream read once (nontemporal hint: no point keeping it in L2)
template <typename T> MTB_DEV void ld8s(const T* p, float (&v)[8]);
template <> MTB_DEV void ld8s<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = lo_f(q[i]); v[2 * i + 1] = hi_f(q[i]); }
}
template <> MTB_DEV void ld8s<float>(const float* p, float (&v)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

// 8 elements of a row as loaded (bf16: one 16-byte word; fp32: two), unpacked later
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
  u32x4 q;
  MTB_DEV void load(const bf16_t* p) { q = *reinterpret_cast<const u32x4*>(p); }
  MTB_DEV void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = lo_f(q[i]); v[2 * i + 1] = hi_f(q[i]); }
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  MTB_DEV void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  MTB_DEV void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
};

// NC = number of 8-element chunks per lane (H <= 512 * NC). Each wavefront
// walks rows row0, row0 + stride, ...; the next row's x (and residual) are
// loaded before the current row is reduced and stored, so that the grid's
// reads and writes overlap instead of running as one burst each.
template <typename T, int NC>
__global__ __launch_bounds__(256) void ln_fwd_kernel(int rows, int H, const T* __restrict__ x,
                                                     const T* __restrict__ resid,
                                                     const T* __restrict__ bias,
                                                     const T* __restrict__ g,
                                                     const T* __restrict__ b, T* __restrict__ h_out,
                                                     T* __restrict__ y, float* __restrict__ mu_out,
                                                     float* __restrict__ rstd_out, float eps,
                                                     Drop drop) {
  const int lane = threadIdx.x & 63;
  const int row0 = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int stride = gridDim.x * kRowsPerBlock;
  Raw8<T> xr[NC], rr[NC];
  auto fetch = [&](int row) {
    const size_t base = (size_t)row * H;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = (c * 64 + lane) * 8;
      if (col < H) {
        xr[c].load(x + base + col);
        if (resid) rr[c].load(resid + base + col);
      }
    }
  };
  if (row0 < rows) fetch(row0);
  for (int row = row0; row < rows; row += stride) {
    const size_t base = (size_t)row * H;
    float v[NC][8];
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = (c * 64 + lane) * 8;
      if (col < H) {
        xr[c].get(v[c]);
        if (resid || bias) {
          // x + dropout(resid + bias)
          float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
          if (resid) rr[c].get(r);
          if (bias) {
            float bb[8];
            ld8(bias + col, bb);
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] += bb[e];
          }
          if (drop.thr) drop_apply8(drop, (uint64_t)base + col, r);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[c][e] += r[e];
          // the stored residual stream and the statistics see the same values
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            T t;
            st_f(&t, v[c][e]);
            v[c][e] = ld_f(&t);
          }
          if (h_out) st8(h_out + base + col, v[c]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s += v[c][e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[c][e] = 0.f;
      }
    }
    if (row + stride < rows) fetch(row + stride);
    const float inv_h = 1.0f / (float)H;
    const float mean = wave_sum(s) * inv_h;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = (c * 64 + lane) * 8;
      if (col < H) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[c][e] - mean;
          q += d * d;
        }
      }
    }
    const float var = wave_sum(q) * inv_h;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = (c * 64 + lane) * 8;
      if (col < H) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (v[c][e] - mean) * rstd;
        if (g) {
          float gg[8], bb[8];
          ld8(g + col, gg);
          ld8(b + col, bb);
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = o[e] * gg[e] + bb[e];
        }
        st8(y + base + col, o);
      }
    }
    if (lane == 0) {
      mu_out[row] = mean;
      rstd_out[row] = rstd;
    }
  }
}

// dx = dres + rstd * (gh - mean(gh) - xhat * mean(gh * xhat)), gh = (dy + dy2) * g;
// dy2 (DY2) and dres (DRES) optional: separate instantiations keep each
// variant's loads straight-line
template <typename T, int NC, bool DY2, bool DRES>
__global__ __launch_bounds__(256) void ln_bwd_kernel(int rows, int H, const T* __restrict__ dy,
                                                     const T* __restrict__ dy2,
                                                     const T* __restrict__ hin,
                                                     const float* __restrict__ mu,
                                                     const float* __restrict__ rstd,
                                                     const T* __restrict__ g,
                                                     const T* __restrict__ dres,
                                                     T* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const size_t base = (size_t)row * H;
  const float m = mu[row], r = rstd[row];
  float gh[NC][8], xh[NC][8];
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = (c * 64 + lane) * 8;
    if (col < H) {
      float hv[8];
      ld8s(dy + base + col, gh[c]);
      if constexpr (DY2) {
        float d2[8];
        ld8s(dy2 + base + col, d2);
#pragma unroll
        for (int e = 0; e < 8; ++e) gh[c][e] += d2[e];
      }
      ld8s(hin + base + col, hv);
      if (g) {
        float gg[8];
        ld8(g + col, gg);
#pragma unroll
        for (int e = 0; e < 8; ++e) gh[c][e] *= gg[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xh[c][e] = (hv[e] - m) * r;
        s1 += gh[c][e];
        s2 += gh[c][e] * xh[c][e];
      }
    }
  }
  const float inv_h = 1.0f / (float)H;
  const float mg = wave_sum(s1) * inv_h;
  const float mgx = wave_sum(s2) * inv_h;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int col = (c * 64 + lane) * 8;
    if (col < H) {
      float o[8], d0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if constexpr (DRES) ld8s(dres + base + col, d0);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = d0[e] + r * (gh[c][e] - mg - xh[c][e] * mgx);
      st8(dx + base + col, o);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_part_kernel(int rows, int N, int rows_per,
                                                          const T* __restrict__ y,
                                                          const T* __restrict__ y2, int ldy,
                                                          const T* __restrict__ hin,
                                                          const float* __restrict__ mu,
                                                          const float* __restrict__ rstd,
                                                          float* __restrict__ part) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  const int r0 = blockIdx.y * rows_per;
  const int r1 = min(rows, r0 + rows_per);
  float acc = 0.f;
  for (int r = r0; r < r1; ++r) {
    float v = ld_f(y + (size_t)r * ldy + n);
    if (y2) v += ld_f(y2 + (size_t)r * ldy + n);
    if (hin) v *= (ld_f(hin + (size_t)r * N + n) - mu[r]) * rstd[r];
    acc += v;
  }
  part[(size_t)blockIdx.y * N + n] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_fin_kernel(int N, int splits,
                                                         const float* __restrict__ part,
                                                         T* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= N) return;
  float acc = 0.f;
  for (int s = 0; s < splits; ++s) acc += part[(size_t)s * N + n];
  st_f(out + n, acc);
}

template <typename T>
__global__ __launch_bounds__(256) void add3_kernel(size_t total8, int H, const T* __restrict__ a,
                                                   const T* __restrict__ b,
                                                   const T* __restrict__ bias,
                                                   T* __restrict__ out, Drop drop) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total8) return;
  const size_t e0 = i * 8;
  float va[8], vb[8];
  ld8(a + e0, va);
  ld8(b + e0, vb);
  if (bias) {
    float vc[8];
    ld8(bias + (int)(e0 % H), vc);
#pragma unroll
    for (int e = 0; e < 8; ++e) vb[e] += vc[e];
  }
  if (drop.thr) drop_apply8(drop, e0, vb);
#pragma unroll
  for (int e = 0; e < 8; ++e) va[e] += vb[e];
  st8(out + e0, va);
}

// out = in * dropout multiplier, element by element (8 per thread)
template <typename T>
__global__ __launch_bounds__(256) void drop_apply_kernel(size_t total8, const T* __restrict__ in,
                                                         T* __restrict__ out, Drop drop) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total8) return;
  float v[8];
  ld8(in + i * 8, v);
  drop_apply8(drop, i * 8, v);
  st8(out + i * 8, v);
}

// GELU: u [rows][F] -> m. SwiGLU: u [rows][2F] (gate/up interleaved by 16) -> m [rows][F].
template <typename T>
__global__ __launch_bounds__(256) void act_fwd_kernel(int act, size_t total, int F,
                                                      const T* __restrict__ u, T* __restrict__ m) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  if (act == 0) {
    st_f(m + i, gelu_f(ld_f(u + i)));
  } else {
    const size_t r = i / F;
    const int f = (int)(i % F);
    const size_t gp = r * 2 * F + (f >> 4) * 32 + (f & 15);
    const float ug = ld_f(u + gp), uu = ld_f(u + gp + 16);
    st_f(m + i, ug * sigmoid_f(ug) * uu);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void act_bwd_kernel(int act, size_t total, int F,
                                                      const T* __restrict__ dm,
                                                      const T* __restrict__ u,
                                                      T* __restrict__ du) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const float d = ld_f(dm + i);
  if (act == 0) {
    st_f(du + i, d * gelu_grad_f(ld_f(u + i)));
  } else {
    const size_t r = i / F;
    const int f = (int)(i % F);
    const size_t gp = r * 2 * F + (f >> 4) * 32 + (f & 15);
    const float ug = ld_f(u + gp), uu = ld_f(u + gp + 16);
    const float s = sigmoid_f(ug);
    st_f(du + gp, d * uu * s * (1.0f + ug * (1.0f - s)));
    st_f(du + gp + 16, d * ug * s);
  }
}

// forward grid: at most LN_FWD_BLOCKS blocks (4 rows of each in flight), so
// that large row counts give each wavefront several rows to pipeline
constexpr int LN_FWD_BLOCKS = 512;

template <typename T, int NC>
hipError_t ln_fwd_t(int rows, int H, const void* x, const void* resid, const void* bias,
                    const void* g, const void* b, void* h_out, void* y, float* mu, float* rstd,
                    float eps, const Drop& drop, hipStream_t st) {
  dim3 grid(std::min((rows + kRowsPerBlock - 1) / kRowsPerBlock, LN_FWD_BLOCKS));
  hipLaunchKernelGGL((ln_fwd_kernel<T, NC>), grid, dim3(256), 0, st, rows, H, (const T*)x,
                     (const T*)resid, (const T*)bias, (const T*)g, (const T*)b, (T*)h_out, (T*)y,
                     mu, rstd, eps, drop);
  return hipGetLastError();
}

template <typename T, int NC>
hipError_t ln_bwd_t(int rows, int H, const void* dy, const void* dy2, const void* hin,
                    const float* mu, const float* rstd, const void* g, const void* dres, void* dx,
                    hipStream_t st) {
  dim3 grid((rows + kRowsPerBlock - 1) / kRowsPerBlock);
#define MTB_LNBK(A2, R)                                                                      \
  hipLaunchKernelGGL((ln_bwd_kernel<T, NC, A2, R>), grid, dim3(256), 0, st, rows, H, (const T*)dy, \
                     (const T*)dy2, (const T*)hin, mu, rstd, (const T*)g, (const T*)dres, (T*)dx)
  if (dy2) {
    if (dres) MTB_LNBK(true, true); else MTB_LNBK(true, false);
  } else {
    if (dres) MTB_LNBK(false, true); else MTB_LNBK(false, false);
  }
#undef MTB_LNBK
  return hipGetLastError();
}

template <typename T>
hipError_t ln_fwd_dispatch(int rows, int H, const void* x, const void* resid, const void* bias,
                           const void* g, const void* b, void* h_out, void* y, float* mu,
                           float* rstd, float eps, const Drop& drop, hipStream_t st) {
  const int nc = (H + 511) / 512;
#define MTB_LNF(N) \
  return ln_fwd_t<T, N>(rows, H, x, resid, bias, g, b, h_out, y, mu, rstd, eps, drop, st)
  if (nc <= 1) MTB_LNF(1);
  if (nc <= 2) MTB_LNF(2);
  if (nc <= 4) MTB_LNF(4);
  if (nc <= 8) MTB_LNF(8);
  if (nc <= 16) MTB_LNF(16);
#undef MTB_LNF
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t ln_bwd_dispatch(int rows, int H, const void* dy, const void* dy2, const void* hin,
                           const float* mu, const float* rstd, const void* g, const void* dres,
                           void* dx, hipStream_t st) {
  const int nc = (H + 511) / 512;
#define MTB_LNB(N) return ln_bwd_t<T, N>(rows, H, dy, dy2, hin, mu, rstd, g, dres, dx, st)
  if (nc <= 1) MTB_LNB(1);
  if (nc <= 2) MTB_LNB(2);
  if (nc <= 4) MTB_LNB(4);
  if (nc <= 8) MTB_LNB(8);
  if (nc <= 16) MTB_LNB(16);
#undef MTB_LNB
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t ln_fwd(int dtype, int rows, int H, const void* x, const void* resid, const void* bias,
                  const void* g, const void* b, void* h_out, void* y, float* mu, float* rstd,
                  float eps, hipStream_t st, const Drop& drop) {
  if (dtype == 1)
    return ln_fwd_dispatch<bf16_t>(rows, H, x, resid, bias, g, b, h_out, y, mu, rstd, eps, drop,
                                   st);
  return ln_fwd_dispatch<float>(rows, H, x, resid, bias, g, b, h_out, y, mu, rstd, eps, drop, st);
}

hipError_t ln_bwd(int dtype, int rows, int H, const void* dy, const void* dy2, const void* hin,
                  const float* mu, const float* rstd, const void* g, const void* dres, void* dx,
                  hipStream_t st) {
  if (dtype == 1)
    return ln_bwd_dispatch<bf16_t>(rows, H, dy, dy2, hin, mu, rstd, g, dres, dx, st);
  return ln_bwd_dispatch<float>(rows, H, dy, dy2, hin, mu, rstd, g, dres, dx, st);
}

int colsum_splits(int rows) { return rows < 64 ? 1 : (rows + 63) / 64 < 128 ? (rows + 63) / 64 : 128; }

hipError_t colsum(int dtype, int rows, int N, const void* y, const void* y2, int ldy,
                  const void* hin, const float* mu, const float* rstd, void* out, float* part,
                  hipStream_t st) {
  const int splits = colsum_splits(rows);
  const int rows_per = (rows + splits - 1) / splits;
  dim3 g1((N + 255) / 256, splits), g2((N + 255) / 256);
  if (dtype == 1) {
    hipLaunchKernelGGL(colsum_part_kernel<bf16_t>, g1, dim3(256), 0, st, rows, N, rows_per,
                       (const bf16_t*)y, (const bf16_t*)y2, ldy, (const bf16_t*)hin, mu, rstd,
                       part);
    hipLaunchKernelGGL(colsum_fin_kernel<bf16_t>, g2, dim3(256), 0, st, N, splits, part,
                       (bf16_t*)out);
  } else {
    hipLaunchKernelGGL(colsum_part_kernel<float>, g1, dim3(256), 0, st, rows, N, rows_per,
                       (const float*)y, (const float*)y2, ldy, (const float*)hin, mu, rstd,
                       part);
    hipLaunchKernelGGL(colsum_fin_kernel<float>, g2, dim3(256), 0, st, N, splits, part,
                       (float*)out);
  }
  return hipGetLastError();
}

hipError_t add3(int dtype, int rows, int H, const void* a, const void* b, const void* bias,
                void* out, hipStream_t st, const Drop& drop) {
  const size_t total8 = (size_t)rows * H / 8;
  dim3 grid((unsigned)((total8 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(add3_kernel<bf16_t>, grid, dim3(256), 0, st, total8, H, (const bf16_t*)a,
                       (const bf16_t*)b, (const bf16_t*)bias, (bf16_t*)out, drop);
  else
    hipLaunchKernelGGL(add3_kernel<float>, grid, dim3(256), 0, st, total8, H, (const float*)a,
                       (const float*)b, (const float*)bias, (float*)out, drop);
  return hipGetLastError();
}

hipError_t drop_apply(int dtype, size_t n, const void* in, void* out, const Drop& drop,
                      hipStream_t st) {
  const size_t total8 = n / 8;
  dim3 grid((unsigned)((total8 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(drop_apply_kernel<bf16_t>, grid, dim3(256), 0, st, total8,
                       (const bf16_t*)in, (bf16_t*)out, drop);
  else
    hipLaunchKernelGGL(drop_apply_kernel<float>, grid, dim3(256), 0, st, total8, (const float*)in,
                       (float*)out, drop);
  return hipGetLastError();
}

hipError_t act_fwd(int dtype, int act, int rows, int F, const void* u, void* m, hipStream_t st) {
  const size_t total = (size_t)rows * F;
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(act_fwd_kernel<bf16_t>, grid, dim3(256), 0, st, act, total, F,
                       (const bf16_t*)u, (bf16_t*)m);
  else
    hipLaunchKernelGGL(act_fwd_kernel<float>, grid, dim3(256), 0, st, act, total, F,
                       (const float*)u, (float*)m);
  return hipGetLastError();
}

hipError_t act_bwd(int dtype, int act, int rows, int F, const void* dm, const void* u, void* du,
                   hipStream_t st) {
  const size_t total = (size_t)rows * F;
  dim3 grid((unsigned)((total + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(act_bwd_kernel<bf16_t>, grid, dim3(256), 0, st, act, total, F,
                       (const bf16_t*)dm, (const bf16_t*)u, (bf16_t*)du);
  else
    hipLaunchKernelGGL(act_bwd_kernel<float>, grid, dim3(256), 0, st, act, total, F,
                       (const float*)dm, (const float*)u, (float*)du);
  return hipGetLastError();
}

}  // namespace mtb
