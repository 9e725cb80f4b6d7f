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
// float64) and rounds each result once to the storage type.  W^K_r sits in LDS
// already widened to float64 and transposed (dimension-major, the 16 outputs of
// one dimension in 128 bytes): all lanes read the same two weights with one
// 16-byte broadcast, and the inner loop holds float64 FMAs only.  Every output
// is one FMA chain over the 128 dimensions in order, which the append path
// repeats, so both give identical bits.  An LDS read returns its bytes to every
// lane, broadcast or not, so the weights' LDS return rate and the float64 FMA
// rate (2048 FMAs per token and head) bound the kernel.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void index_keys_kernel(ProbDev p, const T* __restrict__ k_pre,
                                                              const float* __restrict__ w_k,
                                                              T* __restrict__ k_idx) {
  // w_s[d][j] = W^K_r[j][d] as float64
  __shared__ __attribute__((aligned(16))) double w_s[kHeadDim * kIdxDim];
  const int r = blockIdx.y;
  const float* w = w_k + (size_t)r * kIdxDim * kHeadDim;
  for (int i = threadIdx.x; i < kIdxDim * kHeadDim; i += kThreads) {
    const int j = i / kHeadDim, d = i % kHeadDim;
    w_s[d * kIdxDim + j] = (double)w[i];
  }
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
      const double2* wd = reinterpret_cast<const double2*>(w_s + (d0 + t) * kIdxDim);
#pragma unroll
      for (int j2 = 0; j2 < kIdxDim / 2; ++j2) {
        const double2 wv = wd[j2];
        acc[2 * j2] = fma(xv, wv.x, acc[2 * j2]);
        acc[2 * j2 + 1] = fma(xv, wv.y, acc[2 * j2 + 1]);
      }
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

// ---------------------------------------------------------------- append
// New tokens at the end of every sequence (a decode step appends one): token t
// of sequence b (t = 0 .. n_b - 1) takes position L_b - n_b + t, with L_b the
// length after the append.  Its K and V rows (all KV heads) are copied into the
// cache row of that position - the position itself, or its ring slot when the
// cache keeps only sinks and window - and every retrieval slot gets the index
// key of the new pre-RoPE key, computed exactly as index_keys_kernel does
// (float64 FMA chain over the 128 dims in order, one rounding), so an appended
// cache is bit-identical to one projected in a single pass.  In a ring, tokens
// that no later query can see (neither sinks nor among the last `window`
// positions) are not written, so no two tokens of one call share a slot.
// One workgroup of 128 threads per new token.
template <typename T>
__global__ __launch_bounds__(kHeadDim) void append_kv_kernel(ProbDev p, const int32_t* __restrict__ cu_new,
                                                             int64_t total_new, const T* __restrict__ k_new,
                                                             const T* __restrict__ v_new,
                                                             const T* __restrict__ k_pre_new,
                                                             const float* __restrict__ w_k, T* __restrict__ k,
                                                             T* __restrict__ v, T* __restrict__ k_idx) {
  const int64_t t = blockIdx.x;
  if (t >= total_new) return;
  // sequence of token t: last b with cu_new[b] <= t
  int lo = 0, hi = p.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_new[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int nb = cu_new[b + 1] - cu_new[b];
  const int L = p.cu_k[b + 1] - p.cu_k[b];
  const int pos = L - nb + (int)(t - cu_new[b]);
  if (pos < 0 || pos >= L) return;
  if (p.ring && pos >= p.n_sink && pos < L - p.window) return;   // outside every later window
  const int slot = key_slot(p, pos);
  if (p.kcap > 0 && slot >= p.kcap) return;
  const int64_t row = (int64_t)key_row0(p, b) + slot;
  if (row < 0 || row >= p.Tk) return;
  const int d = threadIdx.x;
  for (int g = 0; g < p.Hkv; ++g) {
    k[((size_t)row * p.Hkv + g) * kHeadDim + d] = k_new[((size_t)t * p.Hkv + g) * kHeadDim + d];
    v[((size_t)row * p.Hkv + g) * kHeadDim + d] = v_new[((size_t)t * p.Hkv + g) * kHeadDim + d];
  }
  // index keys: thread (r, j) over the R * 16 outputs
  for (int o = d; o < p.R * kIdxDim; o += kHeadDim) {
    const int r = o / kIdxDim, j = o % kIdxDim;
    const int g = kv_of(p, p.ret_heads[r]);
    const T* x = k_pre_new + ((size_t)t * p.Hkv + g) * kHeadDim;
    const float* w = w_k + ((size_t)r * kIdxDim + j) * kHeadDim;
    double acc = 0.0;
    for (int e = 0; e < kHeadDim; ++e) acc = fma((double)Elem<T>::to_f(x[e]), (double)w[e], acc);
    k_idx[((size_t)r * p.Tk + row) * kIdxDim + j] = Elem<T>::from_d(acc);
  }
}

}  // namespace

hipError_t launch_append_kv(const ProbDev& p, bool bf16, const int32_t* cu_new, int64_t total_new,
                            const void* k_new, const void* v_new, const void* k_pre_new, const float* w_k,
                            void* k, void* v, void* k_idx, hipStream_t s) {
  if (total_new == 0) return hipSuccess;
  dim3 grid((unsigned)total_new);
  if (bf16)
    hipLaunchKernelGGL(append_kv_kernel<bf16_t>, grid, dim3(kHeadDim), 0, s, p, cu_new, total_new,
                       (const bf16_t*)k_new, (const bf16_t*)v_new, (const bf16_t*)k_pre_new, w_k, (bf16_t*)k,
                       (bf16_t*)v, (bf16_t*)k_idx);
  else
    hipLaunchKernelGGL(append_kv_kernel<float>, grid, dim3(kHeadDim), 0, s, p, cu_new, total_new,
                       (const float*)k_new, (const float*)v_new, (const float*)k_pre_new, w_k, (float*)k,
                       (float*)v, (float*)k_idx);
  return hipGetLastError();
}

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
