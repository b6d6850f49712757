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
// One 256-thread workgroup per token row; 16-byte vector loads when the
// shard width is a multiple of 8 (a scalar loop covers any width).
#include "common.h"
#include "kernels.h"

namespace mtb {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

MTB_DEV void ms_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;  // both empty
  s = (m == kNegInf ? 0.f : s * exp_fast(m - M)) + (m2 == kNegInf ? 0.f : s2 * exp_fast(m2 - M));
  m = M;
}

// block-wide merge of (m, s); result valid in thread 0
MTB_DEV void block_ms(float& m, float& s) {
  __shared__ float sm[4], ss[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    ms_merge(m, s, m2, s2);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[w] = m; ss[w] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < 4; ++i) ms_merge(m, s, sm[i], ss[i]);
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void xent_partial_kernel(int64_t n, int64_t v, int64_t v0,
                                                           const T* __restrict__ z,
                                                           const int64_t* __restrict__ tgt,
                                                           float* __restrict__ stats,
                                                           float* __restrict__ mloc) {
  const int64_t row = blockIdx.x;
  const T* zr = z + row * v;
  float m = kNegInf, s = 0.f;
  if (VEC) {
    for (int64_t c = threadIdx.x; c < v / 8; c += 256) {
      float x[8];
      ld8(zr + c * 8, x);
      float cm = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
      const float M = fmaxf(m, cm);
      float acc = (m == kNegInf) ? 0.f : s * exp_fast(m - M);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += exp_fast(x[e] - M);
      m = M;
      s = acc;
    }
  } else {
    for (int64_t j = threadIdx.x; j < v; j += 256) {
      const float x = ld_f(zr + j);
      const float M = fmaxf(m, x);
      s = ((m == kNegInf) ? 0.f : s * exp_fast(m - M)) + exp_fast(x - M);
      m = M;
    }
  }
  block_ms(m, s);
  if (threadIdx.x == 0) {
    const int64_t lt = tgt[row] - v0;
    const float t = (lt >= 0 && lt < v) ? ld_f(zr + lt) : 0.f;
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
  const int64_t row = blockIdx.x;
  const float M = stats[row], S = stats[n + row];
  if (loss && threadIdx.x == 0) loss[row] = __logf(S) + M - stats[2 * n + row];
  if (!dz) return;
  const float sc = dloss[row] / S;
  const int64_t lt = tgt[row] - v0;
  const T* zr = z + row * v;
  T* dr = dz + row * v;
  if (VEC) {
    for (int64_t c = threadIdx.x; c < v / 8; c += 256) {
      float x[8];
      ld8(zr + c * 8, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = exp_fast(x[e] - M) * sc;
      if (lt >= c * 8 && lt < c * 8 + 8) x[lt - c * 8] -= dloss[row];
      st8(dr + c * 8, x);
    }
  } else {
    for (int64_t j = threadIdx.x; j < v; j += 256) {
      float x = exp_fast(ld_f(zr + j) - M) * sc;
      if (j == lt) x -= dloss[row];
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
  if (v % 8 == 0)
    hipLaunchKernelGGL((xent_partial_kernel<T, true>), dim3((unsigned)n), dim3(256), 0, st, n, v,
                       v0, (const T*)z, tgt, stats, mloc);
  else
    hipLaunchKernelGGL((xent_partial_kernel<T, false>), dim3((unsigned)n), dim3(256), 0, st, n, v,
                       v0, (const T*)z, tgt, stats, mloc);
  return hipGetLastError();
}

template <typename T>
hipError_t finish_t(int64_t n, int64_t v, int64_t v0, const void* z, const int64_t* tgt,
                    const float* stats, float* loss, const float* dloss, void* dz, hipStream_t st) {
  if (v % 8 == 0)
    hipLaunchKernelGGL((xent_finish_kernel<T, true>), dim3((unsigned)n), dim3(dz ? 256 : 64), 0, st,
                       n, v, v0, (const T*)z, tgt, stats, loss, dloss, (T*)dz);
  else
    hipLaunchKernelGGL((xent_finish_kernel<T, false>), dim3((unsigned)n), dim3(dz ? 256 : 64), 0,
                       st, n, v, v0, (const T*)z, tgt, stats, loss, dloss, (T*)dz);
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
