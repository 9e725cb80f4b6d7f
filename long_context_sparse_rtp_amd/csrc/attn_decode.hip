// Decode attention: one query per sequence, exact softmax over a key set.
//
//   retrieval heads: the LIST set chosen by top-p ("Full Attention Strikes
//     Back ...", paper-graph-ui summary, section 3.4, the attention equation
//     that follows Eq. 5: softmax restricted to the selected tokens, post-RoPE
//     q and k, scale 1/sqrt(d_h));
//   local heads: sinks n < n_sink plus the window pos - W < n <= pos
//     (section 3.4 "Local Head Attention Pattern").
//
// The pages' decode kernel ("Hardware-Aware Fast Top-p Decoding Kernel",
// Kernel 2) is bandwidth-bound: single-warp CTAs, registers only, online
// softmax, split-KV with a final merge.  On gfx950 the same bound holds, so
// the kernel is organised for HBM streaming instead of matrix cores:
//   - the set of every (head, sequence) row is cut into splits of 512 entries;
//     the splits of all rows form one flat work list (prefix sums of the
//     per-row split counts, computed on the device) that a fixed grid walks
//     round-robin, so ragged rows and sparse sets leave no idle workgroups;
//   - 16 lanes share a token, each lane holding 8 of the 128 dims, so one K
//     row and one V row are single coalesced 256-byte (bf16) segments; four
//     tokens per 16-lane group are loaded before any arithmetic;
//   - each group keeps an online-softmax state (max, sum, 8 accumulators) in
//     registers; groups merge through LDS, splits merge in a second kernel by
//     log-sum-exp.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;
constexpr int kSplit = 512;
constexpr int kGroups = kThreads / 16;   // 16-lane groups per workgroup
constexpr int kUnroll = 4;
constexpr int kPart = kHeadDim + 2;      // partial record: m, l, o[128]
constexpr int kMaxGrid = 2048;
constexpr int kMaxRowsLds = 4096;        // rows whose split prefix is cached in LDS

struct RowInfo {
  int h, b, qrow, k0, L, count, slot;
};

__device__ __forceinline__ RowInfo row_info(const ProbDev& p, int mode, int row, const rtp_selection& sel) {
  RowInfo ri;
  ri.b = row % p.batch;
  const int hi = row / p.batch;
  ri.k0 = p.cu_k[ri.b];
  ri.L = p.cu_k[ri.b + 1] - ri.k0;
  ri.qrow = p.cu_q[ri.b];
  if (mode == 0) {
    ri.slot = hi;
    ri.h = p.ret_heads[hi];
    ri.count = sel.count[(size_t)hi * p.Tq + ri.qrow];
  } else {
    ri.slot = -1;
    ri.h = p.local_heads[hi];
    const int W = min(p.window, ri.L);
    const int ns = min(p.n_sink, ri.L - W);
    ri.count = ns + W;
  }
  return ri;
}

// j-th key position of a local head's set: sinks first, then the window.
__device__ __forceinline__ int local_token(const ProbDev& p, int L, int j) {
  const int W = min(p.window, L);
  const int ns = min(p.n_sink, L - W);
  return (j < ns) ? j : (L - W + (j - ns));
}

template <typename T> struct RowVec;  // 8 elements of a row
template <> struct RowVec<bf16_t> {
  uint4 raw;
  __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};
template <> struct RowVec<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ float get(int i) const {
    return i < 4 ? (&a.x)[i] : (&b.x)[i - 4];
  }
};

// Split prefix over rows: pre[r] = sum of ceil(count / kSplit) of rows before r; pre[rows] = total.
__global__ __launch_bounds__(1024) void split_prefix_kernel(ProbDev p, int mode, int rows, const rtp_selection sel,
                                                            int* __restrict__ pre) {
  __shared__ int wsum[16];
  __shared__ int carry_s;
  if (threadIdx.x == 0) carry_s = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int base = 0; base < rows; base += 1024) {
    const int r = base + threadIdx.x;
    int v = 0;
    if (r < rows) {
      const RowInfo ri = row_info(p, mode, r, sel);
      v = (ri.count + kSplit - 1) / kSplit;
    }
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d);
      if (lane >= d) inc += y;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int off = carry_s;
    for (int w2 = 0; w2 < wid; ++w2) off += wsum[w2];
    if (r < rows) pre[r] = off + inc - v;
    __syncthreads();
    if (threadIdx.x == 0) {
      int t = 0;
      for (int w2 = 0; w2 < 16; ++w2) t += wsum[w2];
      carry_s += t;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) pre[rows] = carry_s;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(ProbDev p, int mode, int rows, const T* __restrict__ q,
                                                               const T* __restrict__ k, const T* __restrict__ v,
                                                               const rtp_selection sel, const int* __restrict__ pre,
                                                               float* __restrict__ part) {
  __shared__ int pre_s[kMaxRowsLds + 1];
  __shared__ float gm_s[kGroups], gl_s[kGroups];
  __shared__ float go_s[kGroups][kHeadDim];
  const bool lds_pre = rows <= kMaxRowsLds;
  if (lds_pre)
    for (int i = threadIdx.x; i <= rows; i += kThreads) pre_s[i] = pre[i];
  __syncthreads();
  const int total = lds_pre ? pre_s[rows] : pre[rows];
  const int tid = threadIdx.x;
  const int grp = tid >> 4, gl = tid & 15;
  const int d0 = gl * 8;
  const size_t kstride = (size_t)p.Hkv * kHeadDim;
  const float qscale = 0.08838834764831845f * kLog2e;   // log2(e) / sqrt(128)

  for (int wi = blockIdx.x; wi < total; wi += gridDim.x) {
    // row of this work item: last r with pre[r] <= wi
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int pv = lds_pre ? pre_s[mid] : pre[mid];
      if (pv <= wi) lo = mid; else hi = mid - 1;
    }
    const int row = lo;
    const int split = wi - (lds_pre ? pre_s[row] : pre[row]);
    const RowInfo ri = row_info(p, mode, row, sel);
    const int j0 = split * kSplit;
    const int j1 = min(ri.count, j0 + kSplit);
    const int g = kv_of(p, ri.h);
    const T* kb = k + ((size_t)ri.k0 * p.Hkv + g) * kHeadDim + d0;
    const T* vb = v + ((size_t)ri.k0 * p.Hkv + g) * kHeadDim + d0;
    const int* list = (mode == 0) ? sel.idx + (size_t)ri.slot * p.Tk + ri.k0 : nullptr;

    float qv[8];
    {
      RowVec<T> qq;
      qq.load(q + ((size_t)ri.qrow * p.Hq + ri.h) * kHeadDim + d0);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[i] = qq.get(i) * qscale;
    }
    float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.f;

    for (int jb = j0 + grp; jb < j1; jb += kGroups * kUnroll) {
      RowVec<T> kr[kUnroll], vr[kUnroll];
      bool ok[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = jb + u * kGroups;
        ok[u] = j < j1;
        const int n = ok[u] ? ((mode == 0) ? list[j] : local_token(p, ri.L, j)) : 0;
        kr[u].load(kb + (size_t)n * kstride);
        vr[u].load(vb + (size_t)n * kstride);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaf(qv[i], kr[u].get(i), a);
        a += __shfl_xor(a, 1);
        a += __shfl_xor(a, 2);
        a += __shfl_xor(a, 4);
        a += __shfl_xor(a, 8);
        if (ok[u]) {
          const float mn = fmaxf(m, a);
          const float sc = __builtin_amdgcn_exp2f(m - mn);
          const float pe = __builtin_amdgcn_exp2f(a - mn);
          l = l * sc + pe;
#pragma unroll
          for (int i = 0; i < 8; ++i) o[i] = fmaf(pe, vr[u].get(i), o[i] * sc);
          m = mn;
        }
      }
    }

    // merge the 16 groups of the workgroup
    if (gl == 0) { gm_s[grp] = m; gl_s[grp] = l; }
#pragma unroll
    for (int i = 0; i < 8; ++i) go_s[grp][d0 + i] = o[i];
    __syncthreads();
    float* rec = part + (size_t)wi * kPart;
    if (tid < kHeadDim) {
      float M = -INFINITY;
      for (int gi = 0; gi < kGroups; ++gi) M = fmaxf(M, gm_s[gi]);
      float acc = 0.f, sum = 0.f;
      for (int gi = 0; gi < kGroups; ++gi) {
        if (gl_s[gi] > 0.f) {
          const float wgt = __builtin_amdgcn_exp2f(gm_s[gi] - M);
          acc = fmaf(go_s[gi][tid], wgt, acc);
          sum = fmaf(gl_s[gi], wgt, sum);
        }
      }
      rec[2 + tid] = acc;
      if (tid == 0) { rec[0] = M; rec[1] = sum; }
    }
    __syncthreads();
  }
}

// Log-sum-exp merge of a row's split partials: split weights first (one load
// per thread), then every thread sums its head dim over the splits with
// independent loads.
template <typename T>
__global__ __launch_bounds__(kHeadDim) void attn_decode_combine(ProbDev p, int mode, const rtp_selection sel,
                                                                const int* __restrict__ pre,
                                                                const float* __restrict__ part,
                                                                T* __restrict__ out, float* __restrict__ lse) {
  constexpr int kMaxS = 256;
  __shared__ float wgt_s[kMaxS];
  __shared__ float red_s[2];
  __shared__ float sum_s;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const RowInfo ri = row_info(p, mode, row, sel);
  const int s0 = pre[row], s1 = pre[row + 1];
  const int ns = s1 - s0;
  const float* rec = part + (size_t)s0 * kPart;
  float acc = 0.f, M = -INFINITY, sum = 0.f;
  for (int c0 = 0; c0 < ns; c0 += kMaxS) {
    const int cn = min(kMaxS, ns - c0);
    // block max of the split maxima of this chunk
    float mloc = -INFINITY;
    for (int s = tid; s < cn; s += kHeadDim) mloc = fmaxf(mloc, rec[(size_t)(c0 + s) * kPart]);
    mloc = wave_max(mloc);
    if ((tid & 63) == 0) red_s[tid >> 6] = mloc;
    __syncthreads();
    const float mc = fmaxf(red_s[0], red_s[1]);
    const float Mn = fmaxf(M, mc);
    const float scale = __builtin_amdgcn_exp2f(M - Mn);
    acc *= scale;
    sum *= scale;
    M = Mn;
    for (int s = tid; s < cn; s += kHeadDim) {
      const float* rr = rec + (size_t)(c0 + s) * kPart;
      wgt_s[s] = __builtin_amdgcn_exp2f(rr[0] - M);
    }
    __syncthreads();
    if (tid == 0) {
      float sl = 0.f;
      for (int s = 0; s < cn; ++s) sl = fmaf(rec[(size_t)(c0 + s) * kPart + 1], wgt_s[s], sl);
      sum_s = sl;
    }
    int s = 0;
    for (; s + 8 <= cn; s += 8) {
      float v8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v8[u] = rec[(size_t)(c0 + s + u) * kPart + 2 + tid];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc = fmaf(v8[u], wgt_s[s + u], acc);
    }
    for (; s < cn; ++s) acc = fmaf(rec[(size_t)(c0 + s) * kPart + 2 + tid], wgt_s[s], acc);
    __syncthreads();
    sum += sum_s;
    __syncthreads();
  }
  out[((size_t)ri.qrow * p.Hq + ri.h) * kHeadDim + tid] = Elem<T>::from_f(acc / sum);
  if (lse && tid == 0) lse[(size_t)ri.h * p.Tq + ri.qrow] = (M + __log2f(sum)) * 0.6931471805599453f;
}

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// upper bound on the number of splits (every row's set holds at most L_b entries)
inline size_t max_work(const ProbDev& p, int mode, int rows) {
  if (mode == 1) {
    const int cnt = min(p.window, p.max_k) + p.n_sink;
    return (size_t)rows * ((cnt + kSplit - 1) / kSplit);
  }
  const size_t per_row = (size_t)(p.max_k + kSplit - 1) / kSplit;
  const size_t by_total = (size_t)((p.Tk + kSplit - 1) / kSplit) + (size_t)p.batch;  // sum over sequences
  return (size_t)(rows / max(1, p.batch)) * min(per_row * p.batch, by_total);
}

}  // namespace

size_t ws_attn_decode(const ProbDev& p, int mode) {
  const int rows = ((mode == 0) ? p.R : p.n_local) * p.batch;
  return align256(sizeof(int) * (size_t)(rows + 1)) + sizeof(float) * max_work(p, mode, rows) * kPart;
}

hipError_t launch_attn_decode(const ProbDev& p, bool bf16, int mode, const void* q, const void* k,
                              const void* v, const rtp_selection* sel, void* out, float* lse, void* ws,
                              hipStream_t s) {
  const int nheads = (mode == 0) ? p.R : p.n_local;
  if (nheads == 0) return hipSuccess;
  const int rows = nheads * p.batch;
  rtp_selection sl = {};
  if (sel) sl = *sel;
  int* pre = (int*)ws;
  float* part = (float*)((char*)ws + align256(sizeof(int) * (size_t)(rows + 1)));
  hipLaunchKernelGGL(split_prefix_kernel, dim3(1), dim3(1024), 0, s, p, mode, rows, sl, pre);
  const size_t mw = max_work(p, mode, rows);
  const unsigned grid = (unsigned)max((size_t)1, min((size_t)kMaxGrid, mw));
  if (bf16) {
    hipLaunchKernelGGL(attn_decode_kernel<bf16_t>, dim3(grid), dim3(kThreads), 0, s, p, mode, rows, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, sl, (const int*)pre, part);
    hipLaunchKernelGGL(attn_decode_combine<bf16_t>, dim3(rows), dim3(kHeadDim), 0, s, p, mode, sl, (const int*)pre,
                       part, (bf16_t*)out, lse);
  } else {
    hipLaunchKernelGGL(attn_decode_kernel<float>, dim3(grid), dim3(kThreads), 0, s, p, mode, rows, (const float*)q,
                       (const float*)k, (const float*)v, sl, (const int*)pre, part);
    hipLaunchKernelGGL(attn_decode_combine<float>, dim3(rows), dim3(kHeadDim), 0, s, p, mode, sl, (const int*)pre,
                       part, (float*)out, lse);
  }
  return hipGetLastError();
}

}  // namespace rtp
