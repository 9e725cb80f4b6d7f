// Dynamic top-p for one query per sequence (decode), LIST output.
//
// Definition ("Full Attention Strikes Back ...", paper-graph-ui summary,
// section 3.4 "Dynamic Top-p Selection Mechanism", Eq. 5): softmax over the
// indexer scores s_n = q_idx . k_idx_n / 4 of all cached keys, keys taken by
// descending score (ties: ascending position), the smallest prefix whose mass
// reaches p.  Token-exact; the pages' own kernel ("Hardware-Aware Fast Top-p
// Decoding Kernel") approximates with 64-token blocks and a 256-bin
// histogram - kept here only as the idea of a sort-free histogram threshold
// finished by the last workgroup.
//
// Kernel 1 (grid: key chunks x (slot, sequence)): every workgroup projects the
// query (float64, rounded once), scores its 4096-key chunk with the shared
// MFMA indexer tile, writes the float32 scores to the workspace and its chunk
// maximum.  The last workgroup of a row (atomic ticket) then runs the exact
// selection on that row alone:
//   L1  mass histogram of 2048 bins over u = (M - s) log2(e) (64 per octave,
//       last bin open-ended), masses as 32-bit fixed point of 2^(s-M) summed
//       in 64-bit integers (order-independent, so the result is deterministic);
//   scan for the bin where the cumulative mass reaches p * Z;
//   collect that bin's tokens (score, position) - or, if it holds more than
//       1024, refine with radix digits of the score's bit pattern, and finally
//       rank exact ties by position;
//   sort the candidates by (score desc, position asc) and find the crossing
//       token: tau = its score, tie_pos = its position;
//   emit the ascending list {n : s_n > tau or (s_n == tau and n <= tie_pos)}.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;
constexpr int kNB = 2048;        // histogram bins per level
constexpr int kCap = 1024;       // candidate capacity (power of two, bitonic sort)
constexpr float kBinsPerOctave = 64.f;

struct DecodeWs {
  float* scores;       // [R * Tk]
  float* cmax;         // [R * B * max_chunks]
  uint32_t* ticket;    // [R * B]
};

__host__ __device__ inline int max_chunks(const ProbDev& p) { return (p.max_k + kChunk - 1) / kChunk; }

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline DecodeWs carve(const ProbDev& p, void* ws) {
  char* b = (char*)ws;
  DecodeWs w;
  size_t o = 0;
  w.scores = (float*)(b + o);
  o = align256(o + sizeof(float) * (size_t)p.R * p.Tk);
  w.cmax = (float*)(b + o);
  o = align256(o + sizeof(float) * (size_t)p.R * p.batch * max_chunks(p));
  w.ticket = (uint32_t*)(b + o);
  return w;
}

// Per-token quantities every pass of the selection computes the same way.
__device__ __forceinline__ uint32_t mass_fix(float s, float M) {
  const float y = (s - M) * kLog2e;
  const float m = __builtin_amdgcn_exp2f(y);
  return (uint32_t)fminf(m * 4294967296.f, 4294967040.f);
}
__device__ __forceinline__ uint32_t l1_bin(float s, float M) {
  const float y = (s - M) * kLog2e;
  return (uint32_t)fminf(fmaxf(-y * kBinsPerOctave, 0.f), (float)(kNB - 1));
}
// Order-preserving key, descending in s: smaller key = higher score.
__device__ __forceinline__ uint32_t desc_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in s
  return ~u;
}
__device__ __forceinline__ bool is_member(float s, int n, float tau, int tie_pos) {
  return s > tau || (s == tau && n <= tie_pos);
}

// Block-wide exclusive scan of one value per thread (256 threads).
template <typename V>
__device__ V block_exscan(V x, V* tmp /* >= 4 */, V& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  V inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    V y = __shfl_up(inc, d);
    if (lane >= d) inc += y;
  }
  __syncthreads();
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  V off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    if (w < wid) off += tmp[w];
    total += tmp[w];
  }
  return off + inc - x;
}

__global__ void clear_u32(uint32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void select_decode_kernel(
    ProbDev p, const T* __restrict__ q_pre, const float* __restrict__ w_q, const T* __restrict__ k_idx,
    const float* __restrict__ top_p, rtp_selection sel, DecodeWs ws) {
  typedef typename IdxFrag<T>::type IF;
  const int row = blockIdx.y;  // r * batch + b
  const int r = row / p.batch, b = row % p.batch;
  const int k0 = p.cu_k[b];
  const int L = p.cu_k[b + 1] - k0;
  const int nch = (L + kChunk - 1) / kChunk;
  const int c = blockIdx.x;
  if (c >= nch) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int qrow = p.cu_q[b];  // one query per sequence

  __shared__ T q_s[kIdxDim];
  __shared__ float red_s[kThreads / 64];
  __shared__ int last_s;

  // ---- the rounded indexer query (float64, fixed order: every workgroup gets the same bits);
  // the pre-RoPE row and W^Q are staged in LDS first
  {
    __shared__ float wl[kIdxDim * (kHeadDim + 1)];
    __shared__ float xl[kHeadDim];
    for (int e = tid; e < kIdxDim * kHeadDim; e += kThreads)
      wl[(e >> 7) * (kHeadDim + 1) + (e & 127)] = w_q[(size_t)r * kIdxDim * kHeadDim + e];
    if (tid < kHeadDim) xl[tid] = Elem<T>::to_f(q_pre[((size_t)qrow * p.R + r) * kHeadDim + tid]);
    __syncthreads();
    if (tid < kIdxDim) {
      double acc = 0.0;
      for (int d = 0; d < kHeadDim; ++d) acc = fma((double)xl[d], (double)wl[tid * (kHeadDim + 1) + d], acc);
      T qv = Elem<T>::from_d(acc);
      q_s[tid] = qv;
      if (c == 0) ((T*)sel.q_idx)[((size_t)r * p.Tq + qrow) * kIdxDim + tid] = qv;
    }
    __syncthreads();
  }

  // B operand: the query replicated in all 16 columns
  IF qf;
  load_idx_frag(qf, &q_s[4 * (lane >> 4)]);

  // ---- scores of this chunk: 16-key MFMA tiles, waves interleaved
  const T* kbase = k_idx + ((size_t)r * p.Tk + k0) * kIdxDim;
  float* sbase = ws.scores + (size_t)r * p.Tk + k0;
  float tmax = -INFINITY;
  const int n0 = c * kChunk;
  const int nend = min(L, n0 + kChunk);
  for (int t0 = n0 + 16 * wid; t0 < nend; t0 += 16 * (kThreads / 64)) {
    const int key = t0 + (lane & 15);
    IF kf;
    if (key < nend) {
      load_idx_frag(kf, kbase + (size_t)key * kIdxDim + 4 * (lane >> 4));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) kf.v[j] = 0;
    }
    f32x4 acc = idx_dot_tile(kf, qf);
    if ((lane & 15) == 0) {
      const int kb = t0 + 4 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kb + i < nend) {
          const float s = idx_score(acc[i]);
          sbase[kb + i] = s;
          tmax = fmaxf(tmax, s);
        }
      }
    }
  }
  tmax = wave_max(tmax);
  if (lane == 0) red_s[wid] = tmax;
  __threadfence();  // every thread's score stores reach device scope before the ticket
  __syncthreads();
  if (tid == 0) {
    float m = red_s[0];
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red_s[w]);
    ws.cmax[(size_t)row * max_chunks(p) + c] = m;
    __threadfence();
    const uint32_t old = atomicAdd(&ws.ticket[row], 1u);
    last_s = (old == (uint32_t)(nch - 1));
  }
  __syncthreads();
  if (!last_s) return;
  __threadfence();

  // ================= the last workgroup of the row: exact selection
  __shared__ unsigned long long hm_s[kNB];
  __shared__ uint32_t hc_s[kNB];
  __shared__ unsigned long long cand_s[kCap];   // (desc_key(s) << 32) | pos
  __shared__ unsigned long long scan_u64[kThreads / 64];
  __shared__ uint32_t scan_u32[kThreads / 64];
  __shared__ float M_s;
  __shared__ int ncand_s;
  __shared__ unsigned long long above_s;   // fixed-point mass strictly before the chosen bin
  __shared__ uint32_t cabove_s;            // tokens strictly before the chosen bin
  __shared__ int bin_s;
  __shared__ uint32_t bincnt_s;
  __shared__ float tau_s;
  __shared__ int tie_s;
  __shared__ int count_s;

  if (tid == 0) {
    float m = -INFINITY;
    for (int i = 0; i < nch; ++i) m = fmaxf(m, ws.cmax[(size_t)row * max_chunks(p) + i]);
    M_s = m;
  }
  __syncthreads();
  const float M = M_s;
  const float pp = top_p[b];
  const float* sc = ws.scores + (size_t)r * p.Tk + k0;
  int* out_idx = sel.idx + (size_t)r * p.Tk + k0;

  if (!(pp < 1.f)) {  // p >= 1 (or NaN): every key
    for (int n = tid; n < L; n += kThreads) out_idx[n] = n;
    if (tid == 0) {
      sel.count[(size_t)r * p.Tq + qrow] = L;
      if (sel.tau) sel.tau[(size_t)r * p.Tq + qrow] = -INFINITY;
      if (sel.tie_pos) sel.tie_pos[(size_t)r * p.Tq + qrow] = 0x7FFFFFFF;
    }
    return;
  }

  // every pass over the row's scores keeps 8 independent loads in flight per thread
  auto for_scores = [&](auto&& fn) {
    constexpr int U = 8;
    for (int n0 = tid; n0 < L; n0 += U * kThreads) {
      float sv8[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * kThreads;
        sv8[u] = (n < L) ? sc[n] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * kThreads;
        if (n < L) fn(sv8[u], n);
      }
    }
  };

  // ---- L1 histogram
  for (int i = tid; i < kNB; i += kThreads) { hm_s[i] = 0ull; hc_s[i] = 0u; }
  __syncthreads();
  for_scores([&](float s, int n) {
    const uint32_t bin = l1_bin(s, M);
    atomicAdd(&hm_s[bin], (unsigned long long)mass_fix(s, M));
    atomicAdd(&hc_s[bin], 1u);
  });
  __syncthreads();

  // ---- scan: first bin whose inclusive cumulative mass reaches p * Z
  constexpr int kPer = kNB / kThreads;
  unsigned long long lm = 0ull;
  uint32_t lc = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) { lm += hm_s[tid * kPer + j]; lc += hc_s[tid * kPer + j]; }
  unsigned long long Z;
  const unsigned long long pre_m = block_exscan<unsigned long long>(lm, scan_u64, Z);
  uint32_t Ncnt;
  const uint32_t pre_c = block_exscan<uint32_t>(lc, scan_u32, Ncnt);
  const double target = fmax((double)pp * (double)Z, 1.0);
  if ((double)pre_m < target && target <= (double)(pre_m + lm)) {
    unsigned long long cm = pre_m;
    uint32_t cc = pre_c;
    for (int j = 0; j < kPer; ++j) {
      const int bi = tid * kPer + j;
      if ((double)(cm + hm_s[bi]) >= target) {
        bin_s = bi; above_s = cm; cabove_s = cc; bincnt_s = hc_s[bi];
        break;
      }
      cm += hm_s[bi];
      cc += hc_s[bi];
    }
  }
  __syncthreads();
  const int bin1 = bin_s;

  // ---- narrow the candidate set until it fits: radix digits of desc_key(s)
  // within bin1 (levels of 11, 11 and 10 bits); prefix/shift describe the range.
  uint32_t prefix = 0u;
  int shift = 32;          // key bits already fixed: (32 - shift)
  while (bincnt_s > (uint32_t)kCap && shift > 0) {
    const int nbits = (shift >= 11) ? 11 : shift;
    const int nshift = shift - nbits;
    for (int i = tid; i < kNB; i += kThreads) { hm_s[i] = 0ull; hc_s[i] = 0u; }
    __syncthreads();
    for_scores([&](float s, int n) {
      if ((int)l1_bin(s, M) != bin1) return;
      const uint32_t key = desc_key(s);
      if (shift < 32 && (key >> shift) != prefix) return;
      const uint32_t dig = (key >> nshift) & ((1u << nbits) - 1u);
      atomicAdd(&hm_s[dig], (unsigned long long)mass_fix(s, M));
      atomicAdd(&hc_s[dig], 1u);
    });
    __syncthreads();
    if (tid == 0) {
      unsigned long long cm = above_s;
      uint32_t cc = cabove_s;
      for (int d = 0; d < (1 << nbits); ++d) {
        if (hc_s[d] == 0u) continue;
        if ((double)(cm + hm_s[d]) >= target) {
          above_s = cm; cabove_s = cc; bincnt_s = hc_s[d]; bin_s = d;
          break;
        }
        cm += hm_s[d];
        cc += hc_s[d];
      }
    }
    __syncthreads();
    prefix = (shift < 32 ? (prefix << nbits) : 0u) | (uint32_t)bin_s;
    shift = nshift;
  }

  if (bincnt_s > (uint32_t)kCap) {
    // exact ties (identical scores): admit them by ascending position.
    // The tied score value: any token with key == prefix.
    __shared__ float tie_val_s;
    for_scores([&](float s, int n) {
      if ((int)l1_bin(s, M) == bin1 && desc_key(s) == prefix) tie_val_s = s;
    });
    __syncthreads();
    const float tv = tie_val_s;
    const unsigned long long mt = (unsigned long long)mass_fix(tv, M);
    // k = number of tied tokens needed: smallest k with above + k * mt >= target
    const double need = target - (double)above_s;
    long long kneed = (mt > 0) ? (long long)ceil(need / (double)mt) : (long long)bincnt_s;
    if (kneed < 1) kneed = 1;
    if (kneed > (long long)bincnt_s) kneed = bincnt_s;
    // position of the kneed-th tied token: block-wide running count in position order
    __shared__ int tiepos_s;
    __shared__ int run_s;
    if (tid == 0) run_s = 0;
    __syncthreads();
    for (int base = 0; base < L; base += kThreads) {
      const int n = base + tid;
      const uint32_t f = (n < L && sc[n] == tv) ? 1u : 0u;
      uint32_t tot;
      const uint32_t ex = block_exscan<uint32_t>(f, scan_u32, tot);
      const int before = run_s;
      if (f && (long long)(before + ex + 1) == kneed) tiepos_s = n;
      __syncthreads();
      if (tid == 0) run_s = before + (int)tot;
      __syncthreads();
      if ((long long)run_s >= kneed) break;
    }
    if (tid == 0) {
      tau_s = tv;
      tie_s = tiepos_s;
      count_s = (int)cabove_s + (int)kneed;
    }
    __syncthreads();
  } else {
    // ---- collect the candidates of the final bin
    if (tid == 0) ncand_s = 0;
    __syncthreads();
    for_scores([&](float s, int n) {
      if ((int)l1_bin(s, M) != bin1) return;
      if (shift < 32 && (desc_key(s) >> shift) != prefix) return;
      const int slot = atomicAdd(&ncand_s, 1);
      cand_s[slot] = ((unsigned long long)desc_key(s) << 32) | (uint32_t)n;
    });
    __syncthreads();
    const int nc = ncand_s;
    int npow = 64;
    while (npow < nc) npow <<= 1;
    for (int i = nc + tid; i < npow; i += kThreads) cand_s[i] = ~0ull;
    __syncthreads();
    // bitonic sort of the padded candidates, ascending (score desc, position asc)
    for (int k = 2; k <= npow; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < npow; i += kThreads) {
          const int ixj = i ^ j;
          if (ixj > i) {
            const unsigned long long a = cand_s[i], bb = cand_s[ixj];
            const bool up = ((i & k) == 0);
            if ((a > bb) == up) { cand_s[i] = bb; cand_s[ixj] = a; }
          }
        }
        __syncthreads();
      }
    }
    // crossing candidate: 4 consecutive candidates per thread
    unsigned long long cm = 0ull;
    float sv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = tid * 4 + j;
      if (i < nc) {
        const uint32_t kk = (uint32_t)(cand_s[i] >> 32);
        const uint32_t asc = ~kk;
        const uint32_t bits = (asc & 0x80000000u) ? (asc & 0x7FFFFFFFu) : ~asc;
        sv[j] = __uint_as_float(bits);
        cm += mass_fix(sv[j], M);
      } else {
        sv[j] = 0.f;
      }
    }
    unsigned long long tot;
    unsigned long long pre = block_exscan<unsigned long long>(cm, scan_u64, tot) + above_s;
    for (int j = 0; j < 4; ++j) {
      const int i = tid * 4 + j;
      if (i >= nc) break;
      const unsigned long long mj = mass_fix(sv[j], M);
      if ((double)pre < target && (double)(pre + mj) >= target) {
        tau_s = sv[j];
        tie_s = (int)(uint32_t)(cand_s[i] & 0xFFFFFFFFull);
        count_s = (int)cabove_s + i + 1;
        // the candidates hold every token scoring exactly tau: if none is left out, S = {s >= tau}
        if (!(i + 1 < nc && (uint32_t)(cand_s[i + 1] >> 32) == (uint32_t)(cand_s[i] >> 32))) tie_s = 0x7FFFFFFF;
      }
      pre += mj;
    }
    __syncthreads();
  }

  const float tau = tau_s;
  const int tie_pos = tie_s;
  // ---- emit the ascending list: 8 consecutive positions per thread per round
  int run = 0;
  constexpr int E = 8;
  for (int base = 0; base < L; base += E * kThreads) {
    float sv8[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int n = base + E * tid + j;
      sv8[j] = (n < L) ? sc[n] : 0.f;
    }
    uint32_t fl = 0u, lc2 = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int n = base + E * tid + j;
      if (n < L && is_member(sv8[j], n, tau, tie_pos)) { fl |= 1u << j; ++lc2; }
    }
    uint32_t tot2;
    uint32_t ex = block_exscan<uint32_t>(lc2, scan_u32, tot2);
    int o = run + (int)ex;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      if (fl & (1u << j)) out_idx[o++] = base + E * tid + j;
    }
    run += (int)tot2;
  }
  if (tid == 0) {
    sel.count[(size_t)r * p.Tq + qrow] = count_s;
    if (sel.tau) sel.tau[(size_t)r * p.Tq + qrow] = tau;
    if (sel.tie_pos) sel.tie_pos[(size_t)r * p.Tq + qrow] = tie_pos;
  }
}

}  // namespace

size_t ws_select_decode(const ProbDev& p) {
  size_t o = 0;
  o = align256(o + sizeof(float) * (size_t)p.R * p.Tk);
  o = align256(o + sizeof(float) * (size_t)p.R * p.batch * max_chunks(p));
  o = align256(o + sizeof(uint32_t) * (size_t)p.R * p.batch);
  return o;
}

hipError_t launch_select_decode(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                const void* k_idx, const float* top_p, const rtp_selection& sel,
                                void* ws, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  DecodeWs w = carve(p, ws);
  const int nrows = p.R * p.batch;
  hipLaunchKernelGGL(clear_u32, dim3((nrows + 255) / 256), dim3(256), 0, s, w.ticket, nrows);
  dim3 grid(max_chunks(p), nrows);
  if (bf16)
    hipLaunchKernelGGL(select_decode_kernel<bf16_t>, grid, dim3(kThreads), 0, s, p, (const bf16_t*)q_pre,
                       w_q, (const bf16_t*)k_idx, top_p, sel, w);
  else
    hipLaunchKernelGGL(select_decode_kernel<float>, grid, dim3(kThreads), 0, s, p, (const float*)q_pre,
                       w_q, (const float*)k_idx, top_p, sel, w);
  return hipGetLastError();
}

}  // namespace rtp
