// Vocab-parallel cross-entropy on one vocab shard ([TP-block] sec. 4).
//
// The page combines three small reductions over shards: the global row max,
// the target logit (non-zero only on the owning shard) and the sum of
// exponentials. Here one read of the shard's logits gives (m_r, s_r, t_r)
// with an online rescaled sum (s_r = sum exp(z - m_r)), so that after the
// MAX reduction of m the local sum is rescaled by exp(m_r - M) once per row
// instead of re-reading the logits; the three reductions are the same.
// The backward is shard-local: dz = (exp(z - M)/S - onehot) * dloss.
//
// One wavefront per token row, 4 rows per workgroup; 16-byte vector loads
// when the shard width is a multiple of 8 (a scalar loop covers any width).
// Each lane first requests kUnroll chunks of its row (unconditional loads,
// clamped to the row), then reduces them; the row's statistics merge with
// wavefront shuffles only.
#include "common.h"
#include "kernels.h"

namespace mtb {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

MTB_DEV void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;  // both empty
  s = (m == kNegInf ? 0.f : s * exp_fast(m - M)) + (m2 == kNegInf ? 0.f : s2 * exp_fast(m2 - M));
  m = M;
}

constexpr int kUnroll = 8;   // 8-element chunks a thread has in flight

// 8 elements as loaded (bf16: one 16-byte word; fp32: two), unpacked later
template <typename T> struct Raw8;
// (loads with the nontemporal hint: the logits are streamed once per pass)
template <> struct Raw8<bf16_t> {
  u32x4 q;
  MTB_DEV void load(const bf16_t* p) { q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
  MTB_DEV void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[2 * i] = lo_f(q[i]); v[2 * i + 1] = hi_f(q[i]); }
  }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  MTB_DEV void load(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  MTB_DEV void get(float (&v)[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
};

// wavefront-wide merge of (m, s) (every lane ends with the result)
MTB_DEV void wave_ms(float& m, float& s) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
}

// One wavefront per token row (4 rows per workgroup): no block-wide
// reduction, and the target logit is requested before the row's chunks.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void xent_partial_kernel(int64_t n, int64_t v, int64_t v0,
                                                           const T* __restrict__ z,
                                                           const int64_t* __restrict__ tgt,
                                                           float* __restrict__ stats,
                                                           float* __restrict__ mloc) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const T* zr = z + row * v;
  const int64_t lt = tgt[row] - v0;
  const float t = (lt >= 0 && lt < v) ? ld_f(zr + lt) : 0.f;
  float m = kNegInf, s = 0.f;
  if (VEC) {
    const int64_t nch = v / 8;
    for (int64_t base = lane; base < nch; base += 64 * kUnroll) {
      Raw8<T> raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) raw[u].load(zr + min(base + (int64_t)u * 64, nch - 1) * 8);
      float x[kUnroll][8];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) raw[u].get(x[u]);
      // the arithmetic is most of the pass's time: exp(x - M) as
      // exp2(x log2 e - M log2 e), one fma + one v_exp per logit; a batch
      // wholly inside the row runs without per-chunk guards
      const bool whole = base + (int64_t)(kUnroll - 1) * 64 < nch;
      float cm = kNegInf;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (whole || base + (int64_t)u * 64 < nch) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) cm = fmaxf(cm, fmaxf(x[u][e], x[u][e + 1]));
        }
      const float M = fmaxf(m, cm);
      const float Ml = M * kLog2e;
      float acc = (m == kNegInf) ? 0.f : s * exp_fast(m - M);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (whole || base + (int64_t)u * 64 < nch) {
#pragma unroll
          for (int e = 0; e < 8; ++e) acc += __builtin_amdgcn_exp2f(fmaf(x[u][e], kLog2e, -Ml));
        }
      m = M;
      s = acc;
    }
  } else {
    for (int64_t j = lane; j < v; j += 64) {
      const float x = ld_f(zr + j);
      const float M = fmaxf(m, x);
      s = ((m == kNegInf) ? 0.f : s * exp_fast(m - M)) + exp_fast(x - M);
      m = M;
    }
  }
  wave_ms(m, s);
  if (lane == 0) {
    stats[row] = m;
    stats[n + row] = s;
    stats[2 * n + row] = t;
    if (mloc) mloc[row] = m;
  }
}

__global__ __launch_bounds__(256) void xent_rescale_kernel(int64_t n, float* __restrict__ stats,
                                                           const float* __restrict__ mloc) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  stats[n + i] *= exp_fast(mloc[i] - stats[i]);
}

__global__ __launch_bounds__(256) void xent_combine_kernel(int64_t n, int R,
                                                           const float* __restrict__ sh,
                                                           float* __restrict__ stats,
                                                           float* __restrict__ loss) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float M = kNegInf;
  for (int r = 0; r < R; ++r) M = fmaxf(M, sh[(size_t)r * 3 * n + i]);
  float S = 0.f, T = 0.f;
  for (int r = 0; r < R; ++r) {
    const float mr = sh[(size_t)r * 3 * n + i];
    if (mr != kNegInf) S += sh[(size_t)r * 3 * n + n + i] * exp_fast(mr - M);
    T += sh[(size_t)r * 3 * n + 2 * n + i];
  }
  stats[i] = M;
  stats[n + i] = S;
  stats[2 * n + i] = T;
  if (loss) loss[i] = __logf(S) + M - T;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void xent_finish_kernel(int64_t n, int64_t v, int64_t v0,
                                                          const T* __restrict__ z,
                                                          const int64_t* __restrict__ tgt,
                                                          const float* __restrict__ stats,
                                                          float* __restrict__ loss,
                                                          const float* __restrict__ dloss,
                                                          T* __restrict__ dz) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n) return;
  const float M = stats[row], S = stats[n + row];
  if (loss && lane == 0) loss[row] = __logf(S) + M - stats[2 * n + row];
  if (!dz) return;
  const float dl = dloss[row];
  const float sc = dl / S, Ml = M * kLog2e;
  const int64_t lt = tgt[row] - v0;
  const T* zr = z + row * v;
  T* dr = dz + row * v;
  if (VEC) {
    const int64_t nch = v / 8;
    for (int64_t base = lane; base < nch; base += 64 * kUnroll) {
      Raw8<T> raw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) raw[u].load(zr + min(base + (int64_t)u * 64, nch - 1) * 8);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t c = base + (int64_t)u * 64;
        if (c < nch) {
          float x[8];
          raw[u].get(x);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], kLog2e, -Ml)) * sc;
          if (lt >= c * 8 && lt < c * 8 + 8) x[lt - c * 8] -= dl;
          st8(dr + c * 8, x);
        }
      }
    }
  } else {
    for (int64_t j = lane; j < v; j += 64) {
      float x = exp_fast(ld_f(zr + j) - M) * sc;
      if (j == lt) x -= dl;
      st_f(dr + j, x);
    }
  }
}

// per token: merge the (max, sum exp, target logit) of the logits' column
// tiles [n][tiles][3] into stats [3][n] (+ the max into mloc if given); one
// wavefront per token, lanes over the tiles, then a butterfly merge
__global__ __launch_bounds__(256) void lmhead_combine_kernel(int64_t n, int tiles,
                                                             const float* __restrict__ parts,
                                                             float* __restrict__ stats,
                                                             float* __restrict__ mloc) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= n) return;
  const float* p = parts + (size_t)i * tiles * 3;
  float m = kNegInf, s = 0.f, t = 0.f;
  for (int k = lane; k < tiles; k += 64) {
    ms_merge(m, s, p[3 * k], p[3 * k + 1]);
    t += p[3 * k + 2];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
    t += __shfl_xor(t, o, 64);
  }
  if (lane == 0) {
    stats[i] = m;
    stats[n + i] = s;
    stats[2 * n + i] = t;
    if (mloc) mloc[i] = m;
  }
}

template <typename T>
hipError_t partial_t(int64_t n, int64_t v, int64_t v0, const void* z, const int64_t* tgt,
                     float* stats, float* mloc, hipStream_t st) {
  const dim3 grid((unsigned)((n + 3) / 4));
  if (v % 8 == 0)
    hipLaunchKernelGGL((xent_partial_kernel<T, true>), grid, dim3(256), 0, st, n, v, v0, (const T*)z,
                       tgt, stats, mloc);
  else
    hipLaunchKernelGGL((xent_partial_kernel<T, false>), grid, dim3(256), 0, st, n, v, v0, (const T*)z,
                       tgt, stats, mloc);
  return hipGetLastError();
}

template <typename T>
hipError_t finish_t(int64_t n, int64_t v, int64_t v0, const void* z, const int64_t* tgt,
                    const float* stats, float* loss, const float* dloss, void* dz, hipStream_t st) {
  const dim3 grid((unsigned)((n + 3) / 4));
  if (v % 8 == 0)
    hipLaunchKernelGGL((xent_finish_kernel<T, true>), grid, dim3(256), 0, st, n, v, v0, (const T*)z, tgt,
                       stats, loss, dloss, (T*)dz);
  else
    hipLaunchKernelGGL((xent_finish_kernel<T, false>), grid, dim3(256), 0, st, n, v, v0, (const T*)z, tgt,
                       stats, loss, dloss, (T*)dz);
  return hipGetLastError();
}

}  // namespace

hipError_t xent_partial(int dtype, int64_t n, int64_t v, int64_t v0, const void* z,
                        const int64_t* tgt, float* stats, float* mloc, hipStream_t st) {
  return dtype == 1 ? partial_t<bf16_t>(n, v, v0, z, tgt, stats, mloc, st)
                    : partial_t<float>(n, v, v0, z, tgt, stats, mloc, st);
}

hipError_t lmhead_combine(int64_t n, int tiles, const float* parts, float* stats, float* mloc,
                          hipStream_t st) {
  hipLaunchKernelGGL(lmhead_combine_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, st, n,
                     tiles, parts, stats, mloc);
  return hipGetLastError();
}

hipError_t xent_rescale(int64_t n, float* stats, const float* mloc, hipStream_t st) {
  hipLaunchKernelGGL(xent_rescale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n,
                     stats, mloc);
  return hipGetLastError();
}

hipError_t xent_combine(int64_t n, int R, const float* shard_stats, float* stats, float* loss,
                        hipStream_t st) {
  hipLaunchKernelGGL(xent_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, R,
                     shard_stats, stats, loss);
  return hipGetLastError();
}

hipError_t xent_finish(int dtype, int64_t n, int64_t v, int64_t v0, const void* z,
                       const int64_t* tgt, const float* stats, float* loss, const float* dloss,
                       void* dz, hipStream_t st) {
  return dtype == 1 ? finish_t<bf16_t>(n, v, v0, z, tgt, stats, loss, dloss, dz, st)
                    : finish_t<float>(n, v, v0, z, tgt, stats, loss, dloss, dz, st);
}

}  // namespace mtb
