// Vocab-parallel input embedding on one vocab shard ([TP-block] sec. 3).
//
// The [vocab, h] table is split by vocab; this shard holds rows
// [v0, v0 + V). Forward: each token's id is masked to the shard -- in range
// it selects its row, otherwise the token gets a zero row -- and the shards'
// results are summed by the caller's reduction. Backward (the adjoint): the
// replicated output gradient's row of every in-range token is added into its
// id's table row.
//
// Forward: one 256-thread workgroup per token row, 16-byte vectors.
// Backward, deterministically and without a sort: integer atomics give each
// table row its token count and its first token (both independent of the
// order the atomics run in); then one workgroup per table row walks the ids
// from its first token, 256 at a time, lists the matches of each step in
// token order (wavefront ballots), adds their gradient rows in fp32 in that
// order, stops when it has seen the row's count, and writes the row once --
// zeros for a row no token selects.
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "mtb.h"

namespace mtb {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_kernel(int64_t vl, int64_t v0, int H,
                                                        const int64_t* __restrict__ ids,
                                                        const T* __restrict__ table,
                                                        T* __restrict__ out) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte chunk
  const int64_t t = blockIdx.x;
  const int64_t v = ids[t] - v0;
  const bool own = v >= 0 && v < vl;
  const T* src = table + (own ? v : 0) * (size_t)H;
  T* dst = out + (size_t)t * H;
  for (int c = threadIdx.x; c < H / E; c += 256) {
    const u32x4 q = own ? *reinterpret_cast<const u32x4*>(src + c * E) : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(dst + c * E) = q;
  }
}

__global__ __launch_bounds__(256) void embed_init_kernel(int64_t vl, int* __restrict__ cnt,
                                                         int* __restrict__ first) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= vl) return;
  cnt[v] = 0;
  first[v] = 0x7fffffff;
}

__global__ __launch_bounds__(256) void embed_count_kernel(int n, int64_t vl, int64_t v0,
                                                          const int64_t* __restrict__ ids,
                                                          int* __restrict__ cnt,
                                                          int* __restrict__ first) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= n) return;
  const int64_t v = ids[t] - v0;
  if (v < 0 || v >= vl) return;
  atomicAdd(&cnt[v], 1);
  atomicMin(&first[v], t);
}

// CPT 16-byte column chunks per thread per pass over the row's tokens
constexpr int CPT = 4;

template <typename T>
__global__ __launch_bounds__(256) void embed_bwd_kernel(int n, int64_t v0, int H,
                                                        const int64_t* __restrict__ ids,
                                                        const int* __restrict__ cnt,
                                                        const int* __restrict__ first,
                                                        const T* __restrict__ dout,
                                                        T* __restrict__ dtable) {
  __shared__ int hits[256];
  __shared__ int wtot[4];
  const int64_t v = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = cnt[v], t0 = first[v];
  const int64_t gid = v0 + v;
  T* dst = dtable + (size_t)v * H;
  const int H8 = H / 8;
  for (int cg = 0; cg < H8; cg += 256 * CPT) {
    float acc[CPT][8] = {};
    int found = 0;
    // c, found and base are the same in every thread: the loop and its barriers are uniform
    for (int base = t0; found < c; base += 256) {
      const int t = base + tid;
      const bool m = t < n && ids[t] == gid;
      const unsigned long long bal = __ballot(m);
      if (lane == 0) wtot[wave] = __popcll(bal);
      __syncthreads();
      int pos = __popcll(bal & ((1ull << lane) - 1)), nh = 0;
      for (int w = 0; w < 4; ++w) {
        if (w < wave) pos += wtot[w];
        nh += wtot[w];
      }
      if (m) hits[pos] = t;
      __syncthreads();
      for (int h = 0; h < nh; ++h) {
        const int tt = hits[h];
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          const int ch = cg + k * 256 + tid;
          if (ch < H8) {
            float x[8];
            ld8(dout + (size_t)tt * H + ch * 8, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][e] += x[e];
          }
        }
      }
      found += nh;
      __syncthreads();
    }
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      const int ch = cg + k * 256 + tid;
      if (ch < H8) st8(dst + ch * 8, acc[k]);
    }
  }
}

// Device memory of the backward's per-row (count, first token) pairs for
// callers that cannot allocate: one copy per GPU, held until the process
// ends, shared by every call on that GPU (the last call's contents stay).
__device__ __align__(256) int scratch[2 * MTB_EMBED_NOALLOC_MAX_ROWS];

// Its device address on each GPU, looked up once per device with that device
// current. The array's host-side name is not a device address: host code
// uses only these pointers.
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t embed_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t embed_fwd(int dtype, int64_t n, int64_t vl, int64_t v0, int H, const int64_t* ids,
                     const void* table, void* out, hipStream_t st) {
  if (dtype == 1)
    hipLaunchKernelGGL(embed_fwd_kernel<bf16_t>, dim3((unsigned)n), dim3(256), 0, st, vl, v0, H, ids,
                       (const bf16_t*)table, (bf16_t*)out);
  else
    hipLaunchKernelGGL(embed_fwd_kernel<float>, dim3((unsigned)n), dim3(256), 0, st, vl, v0, H, ids,
                       (const float*)table, (float*)out);
  return hipGetLastError();
}

size_t embed_ws_bytes(int64_t vl) { return (size_t)vl * 2 * sizeof(int); }

hipError_t embed_bwd(int dtype, int64_t n, int64_t vl, int64_t v0, int H, const int64_t* ids,
                     const void* dout, void* dtable, void* workspace, hipStream_t st) {
  int* cnt = (int*)workspace;
  int* first = cnt + vl;
  hipLaunchKernelGGL(embed_init_kernel, dim3((unsigned)((vl + 255) / 256)), dim3(256), 0, st, vl, cnt,
                     first);
  hipLaunchKernelGGL(embed_count_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (int)n,
                     vl, v0, ids, cnt, first);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtype == 1)
    hipLaunchKernelGGL(embed_bwd_kernel<bf16_t>, dim3((unsigned)vl), dim3(256), 0, st, (int)n, v0, H,
                       ids, cnt, first, (const bf16_t*)dout, (bf16_t*)dtable);
  else
    hipLaunchKernelGGL(embed_bwd_kernel<float>, dim3((unsigned)vl), dim3(256), 0, st, (int)n, v0, H,
                       ids, cnt, first, (const float*)dout, (float*)dtable);
  return hipGetLastError();
}

}  // namespace mtb
