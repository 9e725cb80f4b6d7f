// Index-key projection: k_idx[r, n, :] = RNE(W^K_r . k_pre[n, kv(ret_heads[r]), :]).
//
// The low-dimensional projection of the pre-RoPE key for each retrieval head
// ("Full Attention Strikes Back ...", paper-graph-ui summary, section 3.4,
// "Low-Dimensional Projection Mechanism": W^K_h in R^{16x128}, applied before
// RoPE).  The cache is what later decode steps score against.
//
// Design: one thread per (token, retrieval head).  The thread streams its
// 256-byte (bf16) key row with 16-byte loads, accumulates the 16 outputs in
// float64 (products of a bf16/f32 element and an f32 weight are exact in
// float64) and rounds each result once to the storage type.  W^K_r (8 KB) sits
// in LDS; all lanes read the same weight at the same time (broadcast).  The
// kernel is bound by HBM reads of k_pre at bf16 and by float64 FMA rate at
// f32; either way it is a small share of a prefill.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void index_keys_kernel(ProbDev p, const T* __restrict__ k_pre,
                                                              const float* __restrict__ w_k,
                                                              T* __restrict__ k_idx) {
  __shared__ float w_s[kIdxDim * kHeadDim];
  const int r = blockIdx.y;
  const float* w = w_k + (size_t)r * kIdxDim * kHeadDim;
  for (int i = threadIdx.x; i < kIdxDim * kHeadDim; i += kThreads) w_s[i] = w[i];
  __syncthreads();

  const int64_t n = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (n >= p.Tk) return;
  const int g = kv_of(p, p.ret_heads[r]);
  const T* x = k_pre + ((size_t)n * p.Hkv + g) * kHeadDim;

  double acc[kIdxDim];
#pragma unroll
  for (int j = 0; j < kIdxDim; ++j) acc[j] = 0.0;

  constexpr int kVec = 16 / sizeof(T);  // elements per 16-byte load
#pragma unroll 2
  for (int d0 = 0; d0 < kHeadDim; d0 += kVec) {
    uint4 raw = *reinterpret_cast<const uint4*>(x + d0);
    const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int t = 0; t < kVec; ++t) {
      const double xv = (double)Elem<T>::to_f(e[t]);
#pragma unroll
      for (int j = 0; j < kIdxDim; ++j) acc[j] = fma(xv, (double)w_s[j * kHeadDim + d0 + t], acc[j]);
    }
  }

  T out[kIdxDim];
#pragma unroll
  for (int j = 0; j < kIdxDim; ++j) out[j] = Elem<T>::from_d(acc[j]);
  uint4* dst = reinterpret_cast<uint4*>(k_idx + ((size_t)r * p.Tk + n) * kIdxDim);
  const uint4* src = reinterpret_cast<const uint4*>(out);
#pragma unroll
  for (int i = 0; i < (int)(kIdxDim * sizeof(T) / 16); ++i) dst[i] = src[i];
}

}  // namespace

hipError_t launch_index_keys(const ProbDev& p, bool bf16, const void* k_pre, const float* w_k,
                             void* k_idx, hipStream_t s) {
  if (p.R == 0 || p.Tk == 0) return hipSuccess;
  dim3 grid((unsigned)((p.Tk + kThreads - 1) / kThreads), p.R);
  if (bf16)
    hipLaunchKernelGGL(index_keys_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p,
                       (const bf16_t*)k_pre, w_k, (bf16_t*)k_idx);
  else
    hipLaunchKernelGGL(index_keys_kernel<float>, grid, dim3(kThreads), 0, s, p, (const float*)k_pre,
                       w_k, (float*)k_idx);
  return hipGetLastError();
}

}  // namespace rtp
