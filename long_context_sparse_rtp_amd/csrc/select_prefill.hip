// Dynamic top-p for every query row of a prefill, THRESHOLD output.
//
// Definition ("Full Attention Strikes Back ...", paper-graph-ui summary,
// section 3.4 "Dynamic Top-p Selection Mechanism", Eq. 5): over the causal
// prefix n <= pos, softmax of s_n = q_idx . k_idx_n / 4, keys by descending
// score (ties: ascending position), the smallest prefix whose mass reaches p.
// The result of a row is (tau, tie_pos, count): S = {s > tau} U {s == tau,
// n <= tie_pos}; tie_pos = INT_MAX when no token scoring exactly tau is left
// out, so that S = {s >= tau}.  Lists are never materialised (a 128K prefill would need
// ~10^10 entries per head).
//
// A workgroup (4 wave64s) owns 16 query rows of one retrieval head; the rows
// are the 16 columns of the shared MFMA indexer tile and the four waves take
// interleaved 16-key tiles of the causal range.  Scores are never stored:
// each sweep over the keys recomputes them with the same MFMA, so every sweep
// (and the attention kernel) sees identical float32 values.
//
// Per token the sweeps use
//   y    = (s - top) * log2(e)   top >= max s (Cauchy-Schwarz bound, or the
//                                 exact row max after a rebase)
//   mass = 2^y as 32-bit fixed point, summed in 64-bit LDS integers (exact,
//          order-independent: results do not depend on wave interleaving)
//   K    = floor(-y * 2^20) saturated to 32 bits (monotone in s)
// Sweep 1 histograms the mass over 256 bins of K >> 16 (16 per octave, the
// last one open-ended) and scans for the bin where the cumulative mass reaches
// p * Z.  Refinement sweeps histogram (mass, count) over the next 8 bits of K
// inside the chosen range until the crossing range holds at most 128 tokens;
// a collect sweep then gathers them, they are sorted by (score desc, position
// asc) and the crossing token gives tau and tie_pos.  Exact ties too large to
// collect switch the key to the score's bit pattern and then to the position.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;
constexpr int kNB = 256;
constexpr int kCap = 128;

enum { PH_HIST1 = 0, PH_REFINE = 1, PH_COLLECT = 2, PH_DONE = 3 };

__device__ __forceinline__ uint32_t desc_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~u;
}

struct RowCtl {
  double target;
  unsigned long long above;   // fixed-point mass of tokens strictly better than the range
  float top;                  // reference score (>= row max)
  float pval;
  uint32_t lo;                // range start in the current key space
  uint32_t kfix, dfix;        // fixed K / desc_key for the tie key spaces
  int sh;                     // digit shift of the range
  int phase, kind;
  int pos;
  float tau;
  int tie, count;
  float smax;
};

__global__ void kidx_norm_clear(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// max over the keys of a sequence of |k_idx|^2 (float bits, non-negative: integer max works)
template <typename T>
__global__ __launch_bounds__(256) void kidx_norm_max(ProbDev p, const T* __restrict__ k_idx,
                                                     uint32_t* __restrict__ out) {
  const int row = blockIdx.y;  // r * batch + b
  const int r = row / p.batch, b = row % p.batch;
  const int k0 = p.cu_k[b], L = p.cu_k[b + 1] - k0;
  float mx = 0.f;
  for (int n = blockIdx.x * 256 + threadIdx.x; n < L; n += gridDim.x * 256) {
    const T* x = k_idx + ((size_t)r * p.Tk + k0 + n) * kIdxDim;
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < kIdxDim; ++j) {
      const float v = Elem<T>::to_f(x[j]);
      a = fmaf(v, v, a);
    }
    mx = fmaxf(mx, a);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) atomicMax(&out[row], __float_as_uint(mx));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void select_prefill_kernel(
    ProbDev p, const T* __restrict__ q_pre, const float* __restrict__ w_q, const T* __restrict__ k_idx,
    const float* __restrict__ top_p, rtp_selection sel, const uint32_t* __restrict__ kn2) {
  typedef typename IdxFrag<T>::type IF;
  const int tiles_per_b = (p.max_q + kRows - 1) / kRows;
  const int b = blockIdx.x / tiles_per_b;
  const int qt = tiles_per_b - 1 - (int)(blockIdx.x % tiles_per_b);  // longest rows first
  const int r = blockIdx.y;
  const int q0 = p.cu_q[b], Lq = p.cu_q[b + 1] - q0;
  const int k0 = p.cu_k[b], Lk = p.cu_k[b + 1] - k0;
  const int i0 = qt * kRows;
  if (i0 >= Lq) return;
  const int off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;

  __shared__ T qidx_s[kRows][kIdxDim];
  __shared__ RowCtl ctl[kRows];
  __shared__ unsigned long long hm_s[kNB][kRows];     // mass, or candidates (aliased)
  __shared__ uint32_t hc_s[kNB][kRows];               // counts
  __shared__ int ccount_s[kRows];
  __shared__ uint32_t cbetter_s[kRows];
  __shared__ float smax_s[4][kRows];
  __shared__ int any_s;
  unsigned long long* cand = &hm_s[0][0];             // [kRows][kCap] during a collect sweep
  static_assert(kRows * kCap <= kNB * kRows, "candidate buffer must fit in the histogram");

  // ---- indexer queries of the 16 rows (float64, fixed order, rounded once)
  {
    const int rr = tid >> 4, j = tid & 15;
    const int i = min(i0 + rr, Lq - 1);
    const T* x = q_pre + ((size_t)(q0 + i) * p.R + r) * kHeadDim;
    const float* wr = w_q + ((size_t)r * kIdxDim + j) * kHeadDim;
    double acc = 0.0;
    for (int d = 0; d < kHeadDim; ++d) acc = fma((double)Elem<T>::to_f(x[d]), (double)wr[d], acc);
    const T qv = Elem<T>::from_d(acc);
    qidx_s[rr][j] = qv;
    if (i0 + rr < Lq) ((T*)sel.q_idx)[((size_t)r * p.Tq + q0 + i0 + rr) * kIdxDim + j] = qv;
  }
  __syncthreads();
  if (tid < kRows) {
    RowCtl& c = ctl[tid];
    const int i = i0 + tid;
    c.pos = (i < Lq) ? off + i : -1;
    c.pval = top_p[b];
    float qn = 0.f;
#pragma unroll
    for (int j = 0; j < kIdxDim; ++j) {
      const float v = Elem<T>::to_f(qidx_s[tid][j]);
      qn = fmaf(v, v, qn);
    }
    const float kn = __uint_as_float(kn2[r * p.batch + b]);
    c.top = sqrtf(qn * kn) * 0.25f * 1.0009765625f + 1e-30f;
    c.above = 0ull;
    c.lo = 0u; c.sh = 16; c.kind = 0; c.kfix = 0u; c.dfix = 0u;
    c.smax = -INFINITY;
    c.tau = -INFINITY; c.tie = 0x7FFFFFFF; c.count = (c.pos >= 0) ? c.pos + 1 : 0;
    c.target = 1.0;
    if (c.pos < 0) {
      c.phase = PH_DONE;
    } else if (!(c.pval < 1.f)) {
      c.phase = PH_DONE;
      c.tau = -INFINITY; c.tie = 0x7FFFFFFF; c.count = c.pos + 1;
    } else {
      c.phase = PH_HIST1;
    }
  }
  __syncthreads();

  IF qxf;
  load_idx_frag(qxf, &qidx_s[col][4 * grp]);
  const T* kxb = k_idx + ((size_t)r * p.Tk + k0) * kIdxDim;
  const int pos_hi = off + min(i0 + kRows, Lq) - 1;
  const int ntile = pos_hi / 16 + 1;

  for (int iter = 0; iter < 64; ++iter) {
    // ---- which kind of sweep: every row taking part is in the same phase, so the
    // candidate buffer can share LDS with the histograms
    if (tid == 0) {
      int k = PH_DONE;
      for (int rr = 0; rr < kRows; ++rr) k = min(k, ctl[rr].phase);
      any_s = k;
    }
    __syncthreads();
    const int sweep = any_s;
    if (sweep == PH_DONE) break;
    const RowCtl c = ctl[col];
    const bool active = (c.phase == sweep);
    // clear the histograms / candidate counters
    for (int e = tid; e < kNB * kRows; e += kThreads) { (&hm_s[0][0])[e] = 0ull; (&hc_s[0][0])[e] = 0u; }
    if (tid < kRows) { ccount_s[tid] = 0; cbetter_s[tid] = 0u; }
    __syncthreads();

    const float c1 = kLog2e * 0.25f;        // y = dot * c1 - top * log2e
    const float c0 = -c.top * kLog2e;
    const int width_sh = (sweep == PH_REFINE) ? (c.sh + 8) : c.sh;
    const int lim = active ? c.pos : -1;    // keys n <= lim take part
    float smax = -INFINITY;
    uint32_t better = 0u;

    for (int t = w; t < ntile; t += 4) {
      const int kb = 16 * t;
      IF kxf;
      const int keyA = kb + col;
      if (keyA < Lk) {
        load_idx_frag(kxf, kxb + (size_t)keyA * kIdxDim + 4 * grp);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) kxf.v[j] = 0;
      }
      const f32x4 dot = idx_dot_tile(kxf, qxf);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = kb + 4 * grp + i;
        if (n > lim) continue;  // causal, and rows not in this sweep
        const float y = fmaf(dot[i], c1, c0);
        const uint32_t K = (uint32_t)__builtin_amdgcn_fmed3f(-y * 1048576.f, 0.f, 4294967040.f);
        if (sweep == PH_HIST1) {
          smax = fmaxf(smax, dot[i]);
          const uint32_t bin = min(K >> 16, (uint32_t)(kNB - 1));
          const float m = __builtin_amdgcn_exp2f(y);
          const uint32_t mf = (uint32_t)fminf(m * 4294967296.f, 4294967040.f);
          atomicAdd(&hm_s[bin][col], (unsigned long long)mf);
          continue;
        }
        uint32_t key = K;
        bool ok = true;
        const float s = idx_score(dot[i]);
        if (c.kind >= 1) {
          const uint32_t dk = desc_key(s);
          ok = (K == c.kfix);
          if (c.kind == 1) {
            key = dk;
          } else {
            ok = ok && (dk == c.dfix);
            key = (uint32_t)n;
          }
          if (sweep == PH_COLLECT) {
            const bool bt = (K < c.kfix) ||
                            (K == c.kfix && (c.kind == 1 ? dk < c.lo
                                                         : (dk < c.dfix || (dk == c.dfix && (uint32_t)n < c.lo))));
            better += bt ? 1u : 0u;
          }
        } else if (sweep == PH_COLLECT) {
          better += (K < c.lo) ? 1u : 0u;
        }
        const uint32_t dk2 = key - c.lo;
        const bool inr = ok && ((width_sh >= 32) ? (key >= c.lo) : ((dk2 >> width_sh) == 0u));
        if (!inr) continue;
        if (sweep == PH_REFINE) {
          const uint32_t dig = dk2 >> c.sh;
          const float m = __builtin_amdgcn_exp2f(y);
          const uint32_t mf = (uint32_t)fminf(m * 4294967296.f, 4294967040.f);
          atomicAdd(&hm_s[dig][col], (unsigned long long)mf);
          atomicAdd(&hc_s[dig][col], 1u);
        } else {
          const int slot = atomicAdd(&ccount_s[col], 1);
          if (slot < kCap) cand[col * kCap + slot] = ((unsigned long long)desc_key(s) << 32) | (uint32_t)n;
        }
      }
    }
    // per-row reductions of this sweep
    if (sweep == PH_HIST1) {
      smax = fmaxf(smax, __shfl_xor(smax, 16));
      smax = fmaxf(smax, __shfl_xor(smax, 32));
      if (grp == 0) smax_s[w][col] = smax;
    }
    if (sweep == PH_COLLECT) {
      better += __shfl_xor(better, 16);
      better += __shfl_xor(better, 32);
      if (grp == 0) atomicAdd(&cbetter_s[col], better);
    }
    __syncthreads();

    // ---- per-row controller
    if (tid < kRows && ctl[tid].phase == sweep) {
      RowCtl& rc = ctl[tid];
      if (rc.phase == PH_HIST1) {
        float sm = fmaxf(fmaxf(smax_s[0][tid], smax_s[1][tid]), fmaxf(smax_s[2][tid], smax_s[3][tid]));
        sm = idx_score(sm);
        if ((sm - rc.top) * kLog2e < -8.f) {
          // loose bound: rebase on the exact row maximum and histogram again
          rc.top = sm;
        } else {
          unsigned long long Z = 0ull;
          for (int bi = 0; bi < kNB; ++bi) Z += hm_s[bi][tid];
          rc.target = fmax((double)rc.pval * (double)Z, 1.0);
          unsigned long long cm = 0ull;
          int bstar = kNB - 1;
          for (int bi = 0; bi < kNB; ++bi) {
            if ((double)(cm + hm_s[bi][tid]) >= rc.target) { bstar = bi; break; }
            cm += hm_s[bi][tid];
          }
          if (bstar == kNB - 1) {  // open-ended last bin: recompute what lies before it
            cm = 0ull;
            for (int bi = 0; bi < kNB - 1; ++bi) cm += hm_s[bi][tid];
          }
          rc.above = cm;
          rc.lo = (uint32_t)bstar << 16;
          rc.sh = (bstar < kNB - 1) ? 8 : 24;   // the last bin spans the rest of the 32-bit key
          rc.phase = PH_REFINE;
        }
      } else if (rc.phase == PH_REFINE) {
        unsigned long long cm = rc.above;
        int dstar = -1;
        uint32_t cnt = 0u;
        for (int d = 0; d < kNB; ++d) {
          if (hc_s[d][tid] == 0u) continue;
          if ((double)(cm + hm_s[d][tid]) >= rc.target) { dstar = d; cnt = hc_s[d][tid]; break; }
          cm += hm_s[d][tid];
        }
        if (dstar < 0) {  // rounding left the target just beyond the range: take its last digit
          cm = rc.above;
          for (int d = 0; d < kNB; ++d) {
            if (hc_s[d][tid] == 0u) continue;
            dstar = d; cnt = hc_s[d][tid];
          }
          for (int d = 0; d < dstar; ++d) cm += hm_s[d][tid];
        }
        rc.above = cm;
        rc.lo = rc.lo + ((uint32_t)dstar << rc.sh);
        if (cnt <= (uint32_t)kCap) {
          rc.phase = PH_COLLECT;
        } else if (rc.sh >= 8) {
          rc.sh -= 8;
        } else if (rc.kind == 0) {
          rc.kind = 1; rc.kfix = rc.lo; rc.lo = 0u; rc.sh = 24;
        } else {
          rc.kind = 2; rc.dfix = rc.lo; rc.lo = 0u; rc.sh = 23;
        }
      } else if (rc.phase == PH_COLLECT) {
        const int nc = min(ccount_s[tid], kCap);
        unsigned long long* cd = cand + tid * kCap;
        for (int a = 1; a < nc; ++a) {  // insertion sort: (desc_key asc, position asc)
          const unsigned long long x = cd[a];
          int bb = a - 1;
          while (bb >= 0 && cd[bb] > x) { cd[bb + 1] = cd[bb]; --bb; }
          cd[bb + 1] = x;
        }
        unsigned long long cm = rc.above;
        int jstar = nc - 1;
        for (int a = 0; a < nc; ++a) {
          const uint32_t kk = ~(uint32_t)(cd[a] >> 32);
          const float s = __uint_as_float((kk & 0x80000000u) ? (kk & 0x7FFFFFFFu) : ~kk);
          const float y = fmaf(s * 4.f, kLog2e * 0.25f, -rc.top * kLog2e);
          const float m = __builtin_amdgcn_exp2f(y);
          const uint32_t mf = (uint32_t)fminf(m * 4294967296.f, 4294967040.f);
          if ((double)(cm + mf) >= rc.target) { jstar = a; break; }
          cm += mf;
        }
        if (nc > 0) {
          const uint32_t kk = ~(uint32_t)(cd[jstar] >> 32);
          rc.tau = __uint_as_float((kk & 0x80000000u) ? (kk & 0x7FFFFFFFu) : ~kk);
          rc.tie = (int)(uint32_t)(cd[jstar] & 0xFFFFFFFFull);
          rc.count = (int)cbetter_s[tid] + jstar + 1;
          // every token scoring exactly tau is a candidate unless the position key was needed;
          // if none of them is left out, the set is simply {s >= tau}
          const bool excluded = (jstar + 1 < nc) && ((uint32_t)(cd[jstar + 1] >> 32) == (uint32_t)(cd[jstar] >> 32));
          if (rc.kind < 2 && !excluded) rc.tie = 0x7FFFFFFF;
        }
        rc.phase = PH_DONE;
      }
    }
    __syncthreads();
  }

  if (tid < kRows && i0 + tid < Lq) {
    const RowCtl& rc = ctl[tid];
    const size_t o = (size_t)r * p.Tq + q0 + i0 + tid;
    sel.tau[o] = rc.tau;
    sel.tie_pos[o] = rc.tie;
    sel.count[o] = rc.count;
  }
}

}  // namespace

size_t ws_select_prefill(const ProbDev& p) { return (sizeof(uint32_t) * (size_t)p.R * p.batch + 255) & ~(size_t)255; }

hipError_t launch_select_prefill(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                 const void* k_idx, const float* top_p, const rtp_selection& sel, void* ws,
                                 hipStream_t s) {
  if (p.R == 0 || p.Tq == 0) return hipSuccess;
  uint32_t* kn2 = (uint32_t*)ws;
  const int nrows = p.R * p.batch;
  hipLaunchKernelGGL(kidx_norm_clear, dim3((nrows + 255) / 256), dim3(256), 0, s, kn2, nrows);
  const int nb = min(64, (p.max_k + 255) / 256);
  if (bf16)
    hipLaunchKernelGGL(kidx_norm_max<bf16_t>, dim3(nb, nrows), dim3(256), 0, s, p, (const bf16_t*)k_idx, kn2);
  else
    hipLaunchKernelGGL(kidx_norm_max<float>, dim3(nb, nrows), dim3(256), 0, s, p, (const float*)k_idx, kn2);
  const int tiles_per_b = (p.max_q + kRows - 1) / kRows;
  dim3 grid(tiles_per_b * p.batch, p.R);
  if (bf16)
    hipLaunchKernelGGL(select_prefill_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p, (const bf16_t*)q_pre, w_q,
                       (const bf16_t*)k_idx, top_p, sel, (const uint32_t*)kn2);
  else
    hipLaunchKernelGGL(select_prefill_kernel<float>, grid, dim3(kThreads), 0, s, p, (const float*)q_pre, w_q,
                       (const float*)k_idx, top_p, sel, (const uint32_t*)kn2);
  return hipGetLastError();
}

}  // namespace rtp
