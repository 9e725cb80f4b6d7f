// Dynamic top-p for one query per sequence (decode), LIST output.
//
// Definition ("Full Attention Strikes Back ...", paper-graph-ui summary,
// section 3.4 "Dynamic Top-p Selection Mechanism", Eq. 5): softmax over the
// indexer scores s_n = q_idx . k_idx_n / 4 of all cached keys, keys taken by
// descending score (ties: ascending position), the smallest prefix whose mass
// reaches p.  Token-exact; the pages' own kernel ("Hardware-Aware Fast Top-p
// Decoding Kernel") approximates with 64-token blocks and a 256-bin histogram
// finished by the last CTA - kept here as the idea of a sort-free histogram
// threshold.  With a top-k budget instead of p (the static top-k the page
// ablates against, sections "Evaluation Methodology" and "Ablation Studies and
// Robustness Checks") the same kernels walk token counts instead of masses:
// the histogram already carries both.
//
// A row (retrieval slot, sequence) is cut into units of 4096 keys.  Two kernels,
// whose boundary is the only synchronisation between workgroups (no device-wide
// fences or tickets):
//
//  1. score, one workgroup per unit: project the query (float64, fixed order,
//     rounded once), score the unit's keys (fixed-order float32 FMA chain), store
//     the scores, and histogram the unit's mass over 4096 bins of 1/128 octave.
//     Bins sit on an absolute grid a(s) = floor(s * 128 * log2(e)); a unit's bin
//     j = A_u - a(s) counts down from the bin A_u of its own maximum, and a
//     token's mass is 38-bit fixed point of 2^(s log2 e - (A_u + 1) / 128).  Mass
//     and count share one 64-bit LDS integer per bin (count << 51), so one atomic
//     per token keeps the sums exact and order-independent.  The fine bins are
//     stored, and so are coarse bins of 16 absolute bins each.
//  2. finish, one workgroup per row: the crossing bin from the units' histograms
//     (unit u's sums scaled by 2^((A_u - A) / 128) in float64, in a fixed order),
//     first the coarse bin where the cumulative mass reaches p * Z, then the fine
//     bin inside it; the bin's tokens from the row's stored scores, ranked by
//     (score desc, position asc) and walked to the crossing token (tau, tie_pos,
//     count); then the members written in ascending order.  A crossing bin too
//     crowded for the candidate buffer (mass piled on near-identical scores) is
//     resolved from the stored scores with radix digits of the score's bit
//     pattern and then positions.
// The finish is bound by the latency of its dependent steps on one compute unit
// (statistics, coarse and fine bins, candidates, ranks, the members' stores), not
// by bandwidth: a row's 128 KB of scores stream through that one unit.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 4096;                  // keys per unit
constexpr int kPer = kChunk / kThreads;       // keys per thread
constexpr int kNB = 4096;                     // bins per unit / row histogram
constexpr int kNC = kNB / 16 + 1;             // coarse bins per unit (16 absolute bins each)
constexpr int kCap = 4096;                    // candidates per row (ranked in LDS)
constexpr int kMaxUnits = 1024;               // units per row (4M keys)
constexpr float kBinScale = 128.f * kLog2e;   // bins per unit of score
constexpr int kCountShift = 51;
constexpr unsigned long long kMassMask = (1ull << kCountShift) - 1ull;

struct UnitMeta {
  int A;                      // absolute bin of the unit maximum
  int used;                   // highest non-empty unit bin (-1: empty unit)
  unsigned long long Z;       // sum of the unit's fixed-point masses
  int cused;                  // highest non-empty coarse bin
};
enum { ROW_NORMAL = 0, ROW_ALL = 1, ROW_EMPTY = 2 };
struct DecodeWs {
  float* scores;               // [R * Tk]
  UnitMeta* meta;              // [nslots]
  unsigned long long* hist;    // [nslots * kNB]
  unsigned long long* chist;   // [nslots * kNC]: 16 absolute bins per coarse bin
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline int max_units(const ProbDev& p) { return (p.max_k + kChunk - 1) / kChunk; }
// Unit slots per retrieval slot: sequence b's units start at cu_k[b] / kChunk + b,
// which leaves room for ceil(L_b / kChunk) units (and one for an empty sequence).
__host__ __device__ inline int64_t slots_per_r(const ProbDev& p) { return p.Tk / kChunk + p.batch + 1; }

inline size_t ws_layout(const ProbDev& p, void* base, DecodeWs* w) {
  const int64_t nslots = (int64_t)p.R * slots_per_r(p);
  char* b = (char*)base;
  size_t o = 0;
  auto take = [&](size_t bytes) { char* q = b ? b + o : nullptr; o = align256(o + bytes); return q; };
  char* s = take(sizeof(float) * (size_t)p.R * p.Tk);
  char* m = take(sizeof(UnitMeta) * nslots);
  char* h = take(sizeof(unsigned long long) * nslots * kNB);
  char* ch = take(sizeof(unsigned long long) * nslots * kNC);
  if (w) {
    w->scores = (float*)s; w->meta = (UnitMeta*)m; w->hist = (unsigned long long*)h;
    w->chist = (unsigned long long*)ch;
  }
  return o;
}

// ---- per-token quantities; every kernel computes them the same way
// absolute bin, clamped to +-2^24 so that bin differences never overflow
__device__ __forceinline__ int abs_bin(float s) {
  return (int)__builtin_amdgcn_fmed3f(floorf(s * kBinScale), -16777216.f, 16777216.f);
}
__device__ __forceinline__ unsigned long long mass38(float s, int A_u) {
  const float e = fminf(fmaf(s, kLog2e, -(float)(A_u + 1) * (1.f / 128.f)), 0.f);
  return (unsigned long long)(__builtin_amdgcn_exp2f(e) * 274877906944.f);   // 2^38
}
__device__ __forceinline__ double unit_scale(int A_u, int A) { return exp2((double)(A_u - A) * (1.0 / 128.0)); }
// Order-preserving key, descending in s: smaller key = higher score.
__device__ __forceinline__ uint32_t desc_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // ascending in s
  return ~u;
}
__device__ __forceinline__ float undesc_key(uint32_t k) {
  const uint32_t a = ~k;
  return __uint_as_float((a & 0x80000000u) ? (a & 0x7FFFFFFFu) : ~a);
}
__device__ __forceinline__ bool is_member(float s, int n, float tau, int tie_pos) {
  return s > tau || (s == tau && n <= tie_pos);
}

struct RowGeom {
  int r, b, row, k0, L, U, qrow;
  int64_t slot0;   // slot of unit 0 of this row
};
__device__ __forceinline__ RowGeom row_geom(const ProbDev& p, int row) {
  RowGeom g;
  g.row = row;
  g.r = row / p.batch;
  g.b = row % p.batch;
  g.k0 = key_row0(p, g.b);
  g.L = p.cu_k[g.b + 1] - p.cu_k[g.b];
  g.U = max(1, (g.L + kChunk - 1) / kChunk);
  g.qrow = p.cu_q[g.b];
  g.slot0 = (int64_t)g.r * slots_per_r(p) + g.k0 / kChunk + g.b;
  return g;
}

// Work order of the score kernel: workgroups are dealt to the 8 XCDs round-robin by
// block id and each XCD has its own L2, so all units of a row go to one XCD (block b:
// k = b / 8, row = 8 (k / U) + b % 8, unit k % U, U unit slots per row).  The finish
// workgroup of a row is block `row`, on XCD row % 8, the same one, so it finds the
// row's histograms and scores in that L2.
__host__ __device__ inline int unit_slots(const ProbDev& p) { return max(1, max_units(p)); }
__host__ __device__ inline unsigned unit_blocks(const ProbDev& p) {
  return 8u * (unsigned)((p.R * p.batch + 7) / 8) * (unsigned)unit_slots(p);
}
__device__ __forceinline__ void unit_of(const ProbDev& p, int b, int& row, int& c) {
  const int U = unit_slots(p);
  const int k = b >> 3;
  row = 8 * (k / U) + (b & 7);
  c = k % U;
}

// ---- block-wide helpers (256 threads, fixed evaluation order)
template <typename V>
__device__ V block_exscan(V x, V* tmp /* >= 4 */, V& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  V inc = wave_scan_add(x);   // inclusive, register-only (DPP)
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
  __syncthreads();
  return off + inc - x;
}
template <typename V>
__device__ V block_max(V x, V* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_allreduce(x, OpMax());
  __syncthreads();
  if (lane == 0) tmp[wid] = x;
  __syncthreads();
  V m = tmp[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = max(m, tmp[w]);
  __syncthreads();
  return m;
}
__device__ double block_sum_f64(double x, double* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_allreduce(x, OpAdd());
  __syncthreads();
  if (lane == 0) tmp[wid] = x;
  __syncthreads();
  const double t = (tmp[0] + tmp[1]) + (tmp[2] + tmp[3]);
  __syncthreads();
  return t;
}
// exclusive float64 scan over the threads (fixed order), plus the total
__device__ double block_exscan_f64(double x, double* tmp, double& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  double inc = wave_scan_add(x);   // inclusive, register-only (DPP)
  __syncthreads();
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wid; ++w) off += tmp[w];
  total = ((tmp[0] + tmp[1]) + tmp[2]) + tmp[3];
  __syncthreads();
  return off + (inc - x);
}

// the same with NW waves (fixed order)
template <int NW>
__device__ double block_exscan_f64_n(double x, double* tmp, double& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  double inc = wave_scan_add(x);   // inclusive, register-only (DPP)
  __syncthreads();
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  double off = 0.0;
  for (int w = 0; w < wid; ++w) off += tmp[w];
  total = 0.0;
  for (int w = 0; w < NW; ++w) total += tmp[w];
  __syncthreads();
  return off + (inc - x);
}

// One key's 16 index values as raw registers, loaded ahead of use.
template <typename T> struct KeyRaw;
template <> struct KeyRaw<bf16_t> {
  uint4 a, b;
  __device__ __forceinline__ void load(const bf16_t* kp) {
    a = reinterpret_cast<const uint4*>(kp)[0];
    b = reinterpret_cast<const uint4*>(kp)[1];
  }
  __device__ __forceinline__ float dot(const float* q) const {
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc = fmaf(q[2 * i], __uint_as_float(w[i] << 16), acc);
      acc = fmaf(q[2 * i + 1], __uint_as_float(w[i] & 0xFFFF0000u), acc);
    }
    return acc;
  }
};
template <> struct KeyRaw<float> {
  float4 v[4];
  __device__ __forceinline__ void load(const float* kp) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const float4*>(kp)[i];
  }
  __device__ __forceinline__ float dot(const float* q) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(q[4 * i], v[i].x, acc);
      acc = fmaf(q[4 * i + 1], v[i].y, acc);
      acc = fmaf(q[4 * i + 2], v[i].z, acc);
      acc = fmaf(q[4 * i + 3], v[i].w, acc);
    }
    return acc;
  }
};

// 8 consecutive elements of a pre-RoPE query row (or of W^Q) as float
__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[2 * i] = __uint_as_float(w[i] << 16); x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u); }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// The rounded indexer query of a decode row: 16 threads per output dim, 8
// products each in float64, combined by a fixed shuffle tree and rounded once.
// Needs all 256 threads; q_s gets the 16 values (visible after a barrier),
// q_out (if not null) too.
template <typename T>
__device__ __forceinline__ void project_query(const ProbDev& p, const RowGeom& g, const T* __restrict__ q_pre,
                                              const float* __restrict__ w_q, T* q_s, T* q_out) {
  const int tid = threadIdx.x;
  const int dim = tid >> 4, part = tid & 15;
  float x[8], wv[8];
  load8(q_pre + ((size_t)g.qrow * p.R + g.r) * kHeadDim + part * 8, x);
  load8(w_q + ((size_t)g.r * kIdxDim + dim) * kHeadDim + part * 8, wv);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = fma((double)x[i], (double)wv[i], acc);
  acc = row16_allreduce(acc, OpAdd());   // the xor 1, 2, 4, 8 tree, register-only
  if (part == 0) {
    const T qv = Elem<T>::from_d(acc);
    q_s[dim] = qv;
    if (q_out) q_out[dim] = qv;
  }
}

// ======================================================================= 1. score
template <typename T>
__global__ __launch_bounds__(kThreads) void sel_dec_score(ProbDev p, const T* __restrict__ q_pre,
                                                          const float* __restrict__ w_q,
                                                          const T* __restrict__ k_idx, rtp_selection sel,
                                                          DecodeWs ws) {
  int row, c;
  unit_of(p, blockIdx.x, row, c);
  if (row >= p.R * p.batch) return;
  const RowGeom g = row_geom(p, row);
  if (c >= g.U || g.U > kMaxUnits) return;
  const int tid = threadIdx.x;
  const int64_t slot = g.slot0 + c;

  __shared__ T q_s[kIdxDim];
  __shared__ unsigned long long hist_s[kNB];
  __shared__ int red_i[kThreads / 64];
  __shared__ unsigned long long red_u[kThreads / 64];


  // keys n = c*kChunk + tid + 256 j: a wave reads consecutive 32/64-byte rows.  The
  // first batch of keys is requested before the query projection so the loads overlap it.
  constexpr int kB = kPer;
  const T* kb = k_idx + ((size_t)g.r * p.Tk + g.k0) * kIdxDim;
  float* sb = ws.scores + (size_t)g.r * p.Tk + g.k0;
  const int n0 = c * kChunk + tid;
  KeyRaw<T> raw[kB];
  auto load_batch = [&](int jb) {
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      const int n = min(n0 + (jb + t) * kThreads, g.L - 1);
      raw[t].load(kb + (size_t)max(n, 0) * kIdxDim);
    }
  };
  if (g.L > 0) load_batch(0);

  // ---- the rounded indexer query
  project_query<T>(p, g, q_pre, w_q, q_s, c == 0 ? (T*)sel.q_idx + ((size_t)g.r * p.Tq + g.qrow) * kIdxDim : nullptr);
  for (int e = tid; e < kNB; e += kThreads) hist_s[e] = 0ull;
  __syncthreads();
  float q[kIdxDim];
#pragma unroll
  for (int d = 0; d < kIdxDim; ++d) q[d] = Elem<T>::to_f(q_s[d]);

  float s[kPer];
  float mx = -INFINITY;
#pragma unroll
  for (int jb = 0; jb < kPer; jb += kB) {
    if (jb > 0 && g.L > 0) load_batch(jb);
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      const int n = n0 + (jb + t) * kThreads;
      s[jb + t] = -INFINITY;
      if (n < g.L) {
        s[jb + t] = idx_score(raw[t].dot(q));
        mx = fmaxf(mx, s[jb + t]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int n = n0 + j * kThreads;
    if (n < g.L) sb[n] = s[j];
  }
  // unit maximum through an order-preserving integer image of the float
  auto ord = [](float f) { const int i = __float_as_int(f); return i ^ ((i >> 31) & 0x7FFFFFFF); };
  const int best = block_max<int>(ord(mx), red_i);
  const bool empty = (g.L == 0) || (c * kChunk >= g.L);
  const float umax = empty ? 0.f : __int_as_float(best ^ ((best >> 31) & 0x7FFFFFFF));
  const int A_u = abs_bin(umax);

  // histogram: one 64-bit atomic per token carries (count << 51) + mass
  unsigned long long zloc = 0ull;
  int used = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int n = n0 + j * kThreads;
    if (n < g.L) {
      const int bin = max(0, min(kNB - 1, A_u - abs_bin(s[j])));
      const unsigned long long m = mass38(s[j], A_u);
      atomicAdd(&hist_s[bin], m | (1ull << kCountShift));
      zloc += m;
      used = max(used, bin);
    }
  }
  unsigned long long Z;
  (void)block_exscan<unsigned long long>(zloc, red_u, Z);
  used = block_max<int>(used, red_i);   // its barriers also order the histogram atomics before the copy
  unsigned long long* hg = ws.hist + slot * kNB;
  for (int e = tid; e <= used; e += kThreads) hg[e] = hist_s[e];
  // coarse bins on the absolute grid: coarse bin cj holds the absolute bins a with
  // a >> 4 == (A_u >> 4) - cj, i.e. unit bins A_u - a
  const int cused = (A_u >> 4) - ((A_u - used) >> 4);
  for (int cj = tid; cj <= cused; cj += kThreads) {
    const int a0 = ((A_u >> 4) - cj) * 16;
    const int jlo = max(A_u - a0 - 15, 0), jhi = min(A_u - a0, used);
    unsigned long long acc = 0ull;
    for (int j = jlo; j <= jhi; ++j) acc += hist_s[j];
    ws.chist[slot * kNC + cj] = acc;
  }
  if (tid == 0) {
    UnitMeta mt;
    mt.A = A_u;
    mt.used = empty ? -1 : used;
    mt.Z = Z;
    mt.cused = empty ? -1 : cused;
    ws.meta[slot] = mt;
  }
}

// ======================================================================= 2. finish
// One workgroup (1024 threads) per row (retrieval slot, sequence) takes the row
// from the units' statistics to its LIST:
//   - the crossing bin: per-unit sums scaled by 2^((A_u - A) / 128) in float64
//     in a fixed order (deterministic), first the coarse row bin where the
//     cumulative mass reaches p * Z, then the fine bin inside it.  Row bins sit
//     on the grid J = Ap - a(s) with Ap = A | 15, A the highest unit bin, so
//     that 16 row bins form one coarse bin of every unit; the last row bin
//     (coarse and fine) is open-ended and holds the row's remainder;
//   - the crossing bin's tokens, gathered from the row's stored scores, which
//     the workgroup holds in registers (32 per thread, chunks of 32K keys),
//     loaded while the crossing is searched;
//   - ranks of those candidates by (score desc, position asc), the walk of
//     their masses to the crossing token (tau, tie_pos, count);
//   - the members written in ascending order: per chunk, one ballot per wave
//     and 64 positions, the wave counts scanned once, then the writes.
// A crossing bin too crowded for the candidate buffer (mass piled on
// near-identical scores) is resolved from the stored scores with radix digits
// of the score's bit pattern and then positions.
constexpr int kRowCoarse = kNB / 16;   // 256 coarse row bins
constexpr int kFT = 1024;              // threads of the finish workgroup
constexpr int kFW = kFT / 64;          // its waves
constexpr int kFS = 32;                // scores per thread per chunk
constexpr int kFChunk = kFS * kFT;     // keys per chunk
static_assert(kMaxUnits <= kFT, "one unit per finish thread");
static_assert(kCap % kFT == 0, "whole ranks per finish thread");

__device__ __forceinline__ double bin_mass(unsigned long long e, double f, bool cmode) {
  return cmode ? (double)(uint32_t)(e >> kCountShift) : (double)(e & kMassMask) * f;
}

// fixed-order block helpers over kFW waves (every thread of the workgroup calls them)
template <typename V>
__device__ V fblock_exscan(V x, V* tmp /* >= kFW */, V& total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  V inc = wave_scan_add(x);   // inclusive, register-only (DPP)
  __syncthreads();
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  V off = 0;
  total = 0;
  for (int w = 0; w < kFW; ++w) {
    if (w < wid) off += tmp[w];
    total += tmp[w];
  }
  __syncthreads();
  return off + (inc - x);
}
__device__ int fblock_max(int x, int* tmp) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_allreduce(x, OpMax());
  __syncthreads();
  if (lane == 0) tmp[wid] = x;
  __syncthreads();
  int m = tmp[0];
  for (int w = 1; w < kFW; ++w) m = max(m, tmp[w]);
  __syncthreads();
  return m;
}

__global__ __launch_bounds__(kFT) void sel_dec_finish(ProbDev p, const float* __restrict__ top_p,
                                                      const int32_t* __restrict__ top_k, rtp_selection sel,
                                                      DecodeWs ws) {
  const int row = blockIdx.x;
  if (row >= p.R * p.batch) return;
  const RowGeom g = row_geom(p, row);
  if (g.U > kMaxUnits) return;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int* out = sel.idx + (size_t)g.r * p.Tk + g.k0;
  const size_t ro = (size_t)g.r * p.Tq + g.qrow;
  const float* sb = ws.scores + (size_t)g.r * p.Tk + g.k0;
  const bool cmode = top_k != nullptr;
  const int nchunks = (g.L + kFChunk - 1) / kFChunk;

  // every unit's statistics and the first chunk of scores are requested before the
  // row's top-p (or k) arrives
  UnitMeta mt = {};
  if (tid < g.U) mt = ws.meta[g.slot0 + tid];
  float sv[kFS];
  // wave w holds positions ch * kFChunk + w * kFS * 64 + 64 i + lane: a contiguous range
  // per wave, so the emission scans kFW wave counts only
  auto pos_of = [&](int ch, int i) { return ch * kFChunk + wid * (kFS * 64) + 64 * i + lane; };
  auto load_chunk = [&](int ch) {
#pragma unroll
    for (int i = 0; i < kFS; ++i) {
      const int n = pos_of(ch, i);
      sv[i] = (n < g.L) ? sb[n] : 0.f;
    }
  };
  load_chunk(0);
  const int kk = cmode ? max(top_k[g.b], 1) : 0;
  const float pp = cmode ? 0.f : top_p[g.b];
  if (g.L == 0 || (cmode ? kk >= g.L : !(pp < 1.f))) {   // empty row; every key (p >= 1 or NaN; k >= L)
    for (int n = tid; n < g.L; n += kFT) out[n] = n;
    if (tid == 0) {
      const bool empty = g.L == 0;
      sel.count[ro] = empty ? 0 : g.L;
      if (sel.tau) sel.tau[ro] = empty ? INFINITY : -INFINITY;
      if (sel.tie_pos) sel.tie_pos[ro] = 0x7FFFFFFF;
    }
    return;
  }

  __shared__ int A_s[kMaxUnits];
  __shared__ int used_s[kMaxUnits];
  __shared__ int cused_s[kMaxUnits];
  __shared__ double f_s[kMaxUnits];
  __shared__ double cm_s[4][kRowCoarse];
  __shared__ uint32_t cc_s[4][kRowCoarse];
  __shared__ double fm_s[kFW][16];
  __shared__ uint32_t fc_s[kFW][16];
  __shared__ double fmt_s[16];
  __shared__ uint32_t fct_s[16];
  __shared__ unsigned long long cand_s[kCap];
  __shared__ short order_s[kCap];
  __shared__ double dtmp[kFW];
  __shared__ int itmp[kFW];
  __shared__ uint32_t utmp[kFW];
  __shared__ int cstar_s, clast_s, jstar_s, js_s, tie_s, count_s, nc_s;
  __shared__ double cab_m_s, cbin_m_s, above_s;
  __shared__ uint32_t cab_c_s, cbin_c_s, cabove_s, bincnt_s;
  __shared__ float tau_s;

  // ---- reference bin A and per-unit scales 2^((A_u - A) / 128); up to 64 units in one
  // wave (shuffle reductions, no block barriers), more with block reductions
  int A;
  double Z;
  if (g.U <= 64) {
    __shared__ int a_sh;
    __shared__ double z_sh;
    if (wid == 0) {
      const bool has = lane < g.U && mt.used >= 0;
      int a = has ? mt.A : (-2147483647 - 1);
      a = wave_allreduce(a, OpMax());
      const double f = has ? unit_scale(mt.A, a) : 0.0;
      double z = (lane < g.U) ? (double)mt.Z * f : 0.0;
      z = wave_allreduce(z, OpAdd());   // the same bits in every lane
      if (lane < g.U) {
        A_s[lane] = mt.A;
        used_s[lane] = mt.used;
        cused_s[lane] = mt.cused;
        f_s[lane] = f;
      }
      if (lane == 0) { a_sh = a; z_sh = z; }
    }
    __syncthreads();
    A = a_sh;
    Z = z_sh;
  } else {
    if (tid < g.U) {
      A_s[tid] = mt.A;
      used_s[tid] = mt.used;
      cused_s[tid] = mt.cused;
    }
    A = fblock_max((tid < g.U && mt.used >= 0) ? mt.A : (-2147483647 - 1), itmp);
    double zl = 0.0;
    if (tid < g.U) {
      const double f = (mt.used >= 0) ? unit_scale(mt.A, A) : 0.0;
      f_s[tid] = f;
      zl = (double)mt.Z * f;
    }
    (void)fblock_exscan<double>(zl, dtmp, Z);   // its barriers also publish A_s, used_s, f_s
  }
  const int Ap = A | 15;
  const double target = cmode ? (double)kk : fmax((double)pp * Z, 1.0);
  // ---- coarse row bins: thread (q, cb) sums units q, q + 4, ... of coarse row bin cb
  {
    const int cb = tid & (kRowCoarse - 1), q = tid >> 8;
    double cm = 0.0;
    uint32_t cc = 0u;
    if (cb < kRowCoarse - 1) {
      for (int u0 = q; u0 < g.U; u0 += 4 * 4) {
        unsigned long long e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int u = u0 + 4 * k;
          e[k] = 0ull;
          if (u < g.U && used_s[u] >= 0) {
            const int cj = cb - ((Ap >> 4) - (A_s[u] >> 4));
            if (cj >= 0 && cj <= cused_s[u]) e[k] = ws.chist[(g.slot0 + u) * kNC + cj];
          }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int u = u0 + 4 * k;
          if (u < g.U) {
            cm += bin_mass(e[k], f_s[u], cmode);
            cc += (uint32_t)(e[k] >> kCountShift);
          }
        }
      }
    }
    cm_s[q][cb] = cm;
    cc_s[q][cb] = cc;
  }
  if (tid == 0) { cstar_s = kRowCoarse; clast_s = -1; nc_s = 0; }
  __syncthreads();
  {
    // one scan gives every coarse bin's prefix and, the last bin holding 0 here, the
    // total of the others: the open-ended last bin is the row's remainder
    double cm = 0.0;
    uint32_t cc = 0u;
    if (tid < kRowCoarse) {
      cm = ((cm_s[0][tid] + cm_s[1][tid]) + cm_s[2][tid]) + cm_s[3][tid];
      cc = ((cc_s[0][tid] + cc_s[1][tid]) + cc_s[2][tid]) + cc_s[3][tid];
    }
    double part;
    uint32_t partc;
    const double pre = fblock_exscan<double>(cm, dtmp, part);
    const uint32_t cpre = fblock_exscan<uint32_t>(cc, utmp, partc);
    if (tid == kRowCoarse - 1) {
      cm = fmax((cmode ? (double)g.L : Z) - part, 0.0);
      cc = (uint32_t)g.L - partc;
    }
    const bool mine = tid < kRowCoarse && cc > 0u;
    if (mine && pre < target && pre + cm >= target) atomicMin(&cstar_s, tid);
    if (mine) atomicMax(&clast_s, tid);
    __syncthreads();
    // rounding left the target just out of reach: the last non-empty coarse bin
    const int cs = (cstar_s < kRowCoarse) ? cstar_s : clast_s;
    if (tid == cs) { cab_m_s = pre; cab_c_s = cpre; cbin_m_s = cm; cbin_c_s = cc; }
    __syncthreads();
    if (tid == 0) cstar_s = cs;
    __syncthreads();
  }
  const int cstar = cstar_s;

  // ---- fine bins of the crossing coarse bin: lane group (i, q) sums units q, q + 64, ...
  {
    const int i = tid & 15, q = tid >> 4;
    const int J = cstar * 16 + i;
    double fm = 0.0;
    uint32_t fc = 0u;
    if (J < kNB - 1) {
      for (int u = q; u < g.U; u += kFT / 16) {
        if (used_s[u] < 0) continue;
        const int j = J - (Ap - A_s[u]);
        if (j >= 0 && j <= used_s[u]) {
          const unsigned long long e = ws.hist[(g.slot0 + u) * kNB + j];
          fm += bin_mass(e, f_s[u], cmode);
          fc += (uint32_t)(e >> kCountShift);
        }
      }
    }
    // lanes i, i + 16, i + 32, i + 48 of a wave hold four groups of bin i
    fm = col4_op(fm, OpAdd());
    fc = col4_op(fc, OpAdd());
    if (lane < 16) { fm_s[wid][i] = fm; fc_s[wid][i] = fc; }
    __syncthreads();
    if (tid < 16) {   // bin tid over the waves, in a fixed order
      double bm = 0.0;
      uint32_t bc = 0u;
      for (int w2 = 0; w2 < kFW; ++w2) { bm += fm_s[w2][tid]; bc += fc_s[w2][tid]; }
      fmt_s[tid] = bm;
      fct_s[tid] = bc;
    }
    __syncthreads();
    if (tid == 0) {
      double m = cab_m_s, rm = cbin_m_s;
      uint32_t cnt = cab_c_s, rc = cbin_c_s;
      int js = -1, jl = -1;
      double ml = 0.0;
      uint32_t cl = 0u, nl = 0u, nb = 0u;
      for (int b2 = 0; b2 < 16; ++b2) {
        double bm = 0.0;
        uint32_t bc = 0u;
        if (cstar * 16 + b2 < kNB - 1) {
          bm = fmt_s[b2];
          bc = fct_s[b2];
          rm -= bm;
          rc -= bc;
        } else {   // the open-ended last bin: what the coarse bin leaves
          bm = fmax(rm, 0.0);
          bc = rc;
        }
        if (bc == 0u) continue;
        if (js < 0 && m + bm >= target) { js = b2; above_s = m; cabove_s = cnt; nb = bc; }
        jl = b2; ml = m; cl = cnt; nl = bc;
        m += bm;
        cnt += bc;
      }
      if (js < 0) { js = jl; above_s = ml; cabove_s = cl; nb = nl; }
      jstar_s = cstar * 16 + js;
      bincnt_s = nb;
    }
    __syncthreads();
  }
  const int jstar = jstar_s;
  auto bin_of = [&](float v) { return min(kNB - 1, Ap - abs_bin(v)); };

  if (bincnt_s <= (uint32_t)kCap) {
    // ---- the crossing bin's tokens from the scores in registers
    for (int ch = 0; ch < nchunks; ++ch) {
      if (ch > 0) load_chunk(ch);
#pragma unroll
      for (int i = 0; i < kFS; ++i) {
        const int n = pos_of(ch, i);
        if (n < g.L && bin_of(sv[i]) == jstar) {
          const int sl = atomicAdd(&nc_s, 1);
          if (sl < kCap) cand_s[sl] = ((unsigned long long)desc_key(sv[i]) << 32) | (uint32_t)n;
        }
      }
    }
    if (nchunks > 1) load_chunk(0);
    __syncthreads();
  }
  const int nc = nc_s;
  if (nc > 0 && nc <= kCap && (uint32_t)nc == bincnt_s) {
    // rank of every candidate in (desc_key, position) order: keys are distinct
    for (int i = tid; i < nc; i += kFT) {
      const unsigned long long ki = cand_s[i];
      int rank = 0;
      for (int j = 0; j < nc; ++j) rank += (cand_s[j] < ki) ? 1 : 0;
      order_s[rank] = (short)i;
    }
    __syncthreads();
    // cumulative masses in rank order: G consecutive ranks per thread, fixed order
    constexpr int G = kCap / kFT;
    double ms[G];
    double loc = 0.0;
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int rk = tid * G + t;
      ms[t] = 0.0;
      if (rk < nc) {
        const unsigned long long kv = cand_s[order_s[rk]];
        const float v = undesc_key((uint32_t)(kv >> 32));
        const int u = min((int)(uint32_t)(kv & 0xFFFFFFFFull) / kChunk, g.U - 1);
        ms[t] = cmode ? 1.0 : (double)mass38(v, A_s[u]) * f_s[u];
      }
      loc += ms[t];
    }
    double tt;
    double pre = fblock_exscan<double>(loc, dtmp, tt) + above_s;
    if (tid == 0) js_s = nc - 1;   // if rounding hides the crossing: the last candidate
    __syncthreads();
#pragma unroll
    for (int t = 0; t < G; ++t) {
      const int rk = tid * G + t;
      pre += ms[t];
      if (rk < nc && pre >= target) { atomicMin(&js_s, rk); break; }
    }
    __syncthreads();
    const int js = js_s;
    if (tid == 0) {
      const unsigned long long kv = cand_s[order_s[js]];
      tau_s = undesc_key((uint32_t)(kv >> 32));
      tie_s = (int)(uint32_t)(kv & 0xFFFFFFFFull);
      // every token scoring exactly tau is a candidate: if none is left out, S = {s >= tau}
      if (!(js + 1 < nc && (uint32_t)(cand_s[order_s[js + 1]] >> 32) == (uint32_t)(kv >> 32))) tie_s = 0x7FFFFFFF;
      count_s = (int)cabove_s + js + 1;
    }
    __syncthreads();
  } else {
    // ---- crowded crossing bin: radix digits of desc_key inside the bin (11 + 11 + 10
    // bits) with masses relative to the row reference, then exact ties by position;
    // the digit histograms share the candidate buffer
    unsigned long long* hm2 = cand_s;
    uint32_t* hc2 = reinterpret_cast<uint32_t*>(cand_s + 2048);
    __shared__ int dig_s, nr_s;
    __shared__ double ab_s;
    __shared__ uint32_t cb_s, cnt_s;
    if (tid == 0) { ab_s = above_s; cb_s = cabove_s; cnt_s = bincnt_s; }
    __syncthreads();
    uint32_t prefix = 0u;
    int shift = 32;
    while (cnt_s > (uint32_t)kCap && shift > 0) {
      const int nbits = (shift >= 11) ? 11 : shift;
      const int nshift = shift - nbits;
      for (int i = tid; i < 2048; i += kFT) { hm2[i] = 0ull; hc2[i] = 0u; }
      __syncthreads();
      for (int n = tid; n < g.L; n += kFT) {
        const float v = sb[n];
        if (bin_of(v) != jstar) continue;
        const uint32_t key = desc_key(v);
        if (shift < 32 && (key >> shift) != prefix) continue;
        const uint32_t dg = (key >> nshift) & ((1u << nbits) - 1u);
        atomicAdd(&hm2[dg], cmode ? 1ull : mass38(v, A));
        atomicAdd(&hc2[dg], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        double cm = ab_s;
        uint32_t cc = cb_s;
        int dsel = -1;
        bool found = false;
        for (int d = 0; d < (1 << nbits); ++d) {
          if (hc2[d] == 0u) continue;
          dsel = d;
          if (cm + (double)hm2[d] >= target) { found = true; break; }
          cm += (double)hm2[d];
          cc += hc2[d];
        }
        if (dsel < 0) dsel = 0;
        if (!found) {  // rounding hid the crossing: the last non-empty digit
          cm = ab_s; cc = cb_s;
          for (int d = 0; d < dsel; ++d) { cm += (double)hm2[d]; cc += hc2[d]; }
        }
        ab_s = cm; cb_s = cc; cnt_s = hc2[dsel]; dig_s = dsel;
      }
      __syncthreads();
      prefix = (shift < 32 ? (prefix << nbits) : 0u) | (uint32_t)dig_s;
      shift = nshift;
    }
    if (cnt_s > (uint32_t)kCap) {
      // exact ties: the tied value is the key `prefix`; admit them by ascending position
      const float tv = undesc_key(prefix);
      const double mt2 = cmode ? 1.0 : (double)mass38(tv, A);
      const double need = target - ab_s;
      long long kneed = (mt2 > 0.0) ? (long long)ceil(need / mt2) : (long long)cnt_s;
      kneed = max(1ll, min(kneed, (long long)cnt_s));
      __shared__ int runt_s, tiepos_s;
      if (tid == 0) { runt_s = 0; tiepos_s = -1; }
      __syncthreads();
      for (int base = 0; base < g.L; base += kFT) {
        const int n = base + tid;
        const uint32_t f = (n < g.L && sb[n] == tv) ? 1u : 0u;
        uint32_t tt2;
        const uint32_t ex = fblock_exscan<uint32_t>(f, utmp, tt2);
        const int before = runt_s;
        if (f && (long long)(before + (int)ex + 1) == kneed) tiepos_s = n;
        __syncthreads();
        if (tid == 0) runt_s = before + (int)tt2;
        __syncthreads();
        if ((long long)runt_s >= kneed) break;
      }
      if (tid == 0) { tau_s = tv; tie_s = tiepos_s; count_s = (int)cb_s + (int)kneed; }
      __syncthreads();
    } else {
      // the remaining range fits: collect it, rank it and walk it
      if (tid == 0) nr_s = 0;
      __syncthreads();
      for (int n = tid; n < g.L; n += kFT) {
        const float v = sb[n];
        if (bin_of(v) != jstar) continue;
        if (shift < 32 && (desc_key(v) >> shift) != prefix) continue;
        const int sl = atomicAdd(&nr_s, 1);
        if (sl < kCap) cand_s[sl] = ((unsigned long long)desc_key(v) << 32) | (uint32_t)n;
      }
      __syncthreads();
      const int nr = min(nr_s, kCap);
      for (int i = tid; i < nr; i += kFT) {
        const unsigned long long ki = cand_s[i];
        int rank = 0;
        for (int j = 0; j < nr; ++j) rank += (cand_s[j] < ki) ? 1 : 0;
        order_s[rank] = (short)i;
      }
      __syncthreads();
      if (tid == 0) {
        double cm = ab_s;
        int js = max(nr - 1, 0);
        for (int i = 0; i < nr; ++i) {
          const float v = undesc_key((uint32_t)(cand_s[order_s[i]] >> 32));
          const double mi = cmode ? 1.0 : (double)mass38(v, A);
          if (cm + mi >= target) { js = i; break; }
          cm += mi;
        }
        const unsigned long long kv = cand_s[order_s[js]];
        tau_s = undesc_key((uint32_t)(kv >> 32));
        tie_s = (int)(uint32_t)(kv & 0xFFFFFFFFull);
        if (!(js + 1 < nr && (uint32_t)(cand_s[order_s[js + 1]] >> 32) == (uint32_t)(kv >> 32))) tie_s = 0x7FFFFFFF;
        count_s = (int)cb_s + js + 1;
      }
      __syncthreads();
    }
  }

  // ---- the members, ascending: per chunk, a ballot per (step, wave) of 64 positions,
  // the ballot counts scanned in position order, then the writes
  const float tau = tau_s;
  const int tie = tie_s;
  if (tid == 0) {
    sel.count[ro] = count_s;
    if (sel.tau) sel.tau[ro] = tau;
    if (sel.tie_pos) sel.tie_pos[ro] = tie;
  }
  const unsigned long long below = (1ull << lane) - 1ull;
  uint32_t run = 0u;   // members of the chunks before
  for (int ch = 0; ch < nchunks; ++ch) {
    if (ch > 0) load_chunk(ch);
    // the wave's members: one bit per step in a lane register, and their count
    uint32_t bits = 0u, wc = 0u;
#pragma unroll
    for (int i = 0; i < kFS; ++i) {
      const int n = pos_of(ch, i);
      const bool m = n < g.L && is_member(sv[i], n, tau, tie);
      bits |= m ? (1u << i) : 0u;
      wc += (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(m));
    }
    if (lane == 0) utmp[wid] = wc;
    __syncthreads();
    uint32_t o = run, ctot = 0u;
    for (int w2 = 0; w2 < kFW; ++w2) {
      const uint32_t c = utmp[w2];
      if (w2 < wid) o += c;
      ctot += c;
    }
#pragma unroll
    for (int i = 0; i < kFS; ++i) {
      const unsigned long long mk = __builtin_amdgcn_ballot_w64((bits >> i) & 1u);
      if ((bits >> i) & 1u) {
        const uint32_t at = o + (uint32_t)__popcll(mk & below);
        if (at < (uint32_t)g.L) out[at] = pos_of(ch, i);
      }
      o += (uint32_t)__popcll(mk);
    }
    run += ctot;
    __syncthreads();
  }
}

// ======================================================================= block top-p
// The pages' own decode selection ("Hardware-Aware Fast Top-p Decoding
// Kernel", steps 1-5): 64-token blocks reduced to (max score m_b, block mass),
// block masses binned by m_b over 256 equal bins of the row's [min m_b,
// max m_b], bins scanned from the top to the first where the cumulative
// fraction reaches p, every block in that bin or above kept whole.  The
// selection is written as a LIST of the kept blocks' positions, so the decode
// attention consumes it unchanged.  Two kernels: block statistics with one
// workgroup per unit of 4096 keys (the pages use one CTA per block; a wave
// per block keeps the whole device busy with 256-thread workgroups), then one
// workgroup per row for the histogram, the scan and the list.
constexpr int kBlk = 64;
constexpr int kBlkBins = 256;

// Block statistics of sequence b, slot r start here: room for ceil(L_b / 64) blocks.
__host__ __device__ inline int64_t blk_slots_per_r(const ProbDev& p) { return p.Tk / kBlk + p.batch + 1; }
__device__ __forceinline__ int64_t blk_slot0(const ProbDev& p, const RowGeom& g) {
  return (int64_t)g.r * blk_slots_per_r(p) + g.k0 / kBlk + g.b;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void sel_blk_score(ProbDev p, const T* __restrict__ q_pre,
                                                          const float* __restrict__ w_q,
                                                          const T* __restrict__ k_idx, rtp_selection sel,
                                                          float2* __restrict__ bstat) {
  const RowGeom g = row_geom(p, blockIdx.y);
  const int c = blockIdx.x;
  if (c >= g.U || g.U > kMaxUnits || g.L == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  __shared__ T q_s[kIdxDim];

  // keys n = c*kChunk + tid + 256 j: wave w of step j holds block c*64 + 4 j + w
  const T* kb = k_idx + ((size_t)g.r * p.Tk + g.k0) * kIdxDim;
  const int n0 = c * kChunk + tid;
  KeyRaw<T> raw[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) raw[j].load(kb + (size_t)min(n0 + j * kThreads, g.L - 1) * kIdxDim);
  project_query<T>(p, g, q_pre, w_q, q_s, c == 0 ? (T*)sel.q_idx + ((size_t)g.r * p.Tq + g.qrow) * kIdxDim : nullptr);
  __syncthreads();
  float q[kIdxDim];
#pragma unroll
  for (int d = 0; d < kIdxDim; ++d) q[d] = Elem<T>::to_f(q_s[d]);

  float2* bs = bstat + blk_slot0(p, g);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int n = n0 + j * kThreads;
    const bool valid = n < g.L;
    const float sc = valid ? idx_score(raw[j].dot(q)) : -INFINITY;
    const float m = wave_max(sc);
    const float e = valid ? __builtin_amdgcn_exp2f((sc - m) * kLog2e) : 0.f;
    const float l = wave_sum(e);
    const int blk = c * (kChunk / kBlk) + 4 * j + w;
    if (lane == 0 && blk * kBlk < g.L) bs[blk] = make_float2(m, l);
  }
}

__global__ __launch_bounds__(kThreads) void sel_blk_choose(ProbDev p, const float* __restrict__ top_p,
                                                           rtp_selection sel, const float2* __restrict__ bstat) {
  const RowGeom g = row_geom(p, blockIdx.x);
  const int tid = threadIdx.x;
  const size_t qo = (size_t)g.r * p.Tq + g.qrow;
  if (g.L == 0) {
    if (tid == 0) {
      sel.count[qo] = 0;
      if (sel.tau) sel.tau[qo] = INFINITY;
      if (sel.tie_pos) sel.tie_pos[qo] = 0x7FFFFFFF;
    }
    return;
  }
  __shared__ unsigned long long hist_s[kBlkBins];
  __shared__ unsigned long long red_u[kThreads / 64];
  __shared__ int red_i[kThreads / 64];
  __shared__ uint32_t utmp[kThreads / 64];
  __shared__ uint32_t offs_s[kThreads];
  __shared__ int jstar_s;
  const int nb = (g.L + kBlk - 1) / kBlk;
  const float2* bs = bstat + blk_slot0(p, g);

  // ---- range of the block maxima (order-preserving integer images of the floats)
  auto ord = [](float f) { const int i = __float_as_int(f); return i ^ ((i >> 31) & 0x7FFFFFFF); };
  auto unord = [](int i) { return __int_as_float(i ^ ((i >> 31) & 0x7FFFFFFF)); };
  float hi = -INFINITY, nlo = -INFINITY;
  for (int i = tid; i < nb; i += kThreads) {
    const float m = bs[i].x;
    hi = fmaxf(hi, m);
    nlo = fmaxf(nlo, -m);
  }
  hi = unord(block_max<int>(ord(hi), red_i));
  const float lo = -unord(block_max<int>(ord(nlo), red_i));
  const bool spread = hi > lo;
  const float scale = spread ? (float)kBlkBins / (hi - lo) : 0.f;
  auto bin_of = [&](float m) { return spread ? min(kBlkBins - 1, (int)((m - lo) * scale)) : kBlkBins - 1; };

  // ---- block masses relative to the row maximum, 2^32 fixed point (a block holds at most 2^38)
  for (int e = tid; e < kBlkBins; e += kThreads) hist_s[e] = 0ull;
  __syncthreads();
  for (int i = tid; i < nb; i += kThreads) {
    const float2 v = bs[i];
    const float mf = v.y * __builtin_amdgcn_exp2f((v.x - hi) * kLog2e) * 4294967296.f;
    atomicAdd(&hist_s[bin_of(v.x)], (unsigned long long)mf);
  }
  __syncthreads();

  // ---- the crossing bin: thread t holds bin 255 - t, so the exclusive scan is the mass above it
  const float pp = top_p[g.b];
  const bool all = !(pp < 1.f);
  if (tid == 0) jstar_s = 0;
  const unsigned long long h = hist_s[kBlkBins - 1 - tid];
  unsigned long long tot;
  const unsigned long long pre = block_exscan<unsigned long long>(h, red_u, tot);
  if (!all) {
    const unsigned long long tgt = (unsigned long long)ceil((double)pp * (double)tot);
    const unsigned long long need = tgt > 0ull ? tgt : 1ull;
    if (pre < need && need <= pre + h) jstar_s = kBlkBins - 1 - tid;
  }
  __syncthreads();
  const int jstar = jstar_s;

  // ---- the kept blocks' positions, ascending: 256 blocks at a time, one per thread
  int* out = sel.idx + (size_t)g.r * p.Tk + g.k0;
  uint32_t base = 0u;
  for (int c0 = 0; c0 < nb; c0 += kThreads) {
    const int i = c0 + tid;
    const bool keep = i < nb && bin_of(bs[i].x) >= jstar;
    const uint32_t len = keep ? (uint32_t)min(kBlk, g.L - i * kBlk) : 0u;
    uint32_t ctot;
    const uint32_t off = block_exscan<uint32_t>(len, utmp, ctot);
    offs_s[tid] = keep ? base + off : 0xFFFFFFFFu;
    __syncthreads();
    for (int e = tid; e < kThreads * kBlk; e += kThreads) {
      const uint32_t o = offs_s[e / kBlk];
      const int n = (c0 + e / kBlk) * kBlk + (e % kBlk);
      if (o != 0xFFFFFFFFu && n < g.L) out[o + (e % kBlk)] = n;
    }
    base += ctot;
    __syncthreads();
  }
  if (tid == 0) {
    sel.count[qo] = (int)base;
    if (sel.tau) sel.tau[qo] = all ? -INFINITY : (spread ? lo + (float)jstar / scale : lo);
    if (sel.tie_pos) sel.tie_pos[qo] = 0x7FFFFFFF;
  }
}

}  // namespace

size_t ws_select_decode(const ProbDev& p) { return ws_layout(p, nullptr, nullptr); }

hipError_t launch_select_decode(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                const void* k_idx, const float* top_p, const int32_t* top_k,
                                const rtp_selection& sel, void* ws, hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  DecodeWs w;
  ws_layout(p, ws, &w);
  const dim3 grid(unit_blocks(p));
  if (bf16)
    hipLaunchKernelGGL(sel_dec_score<bf16_t>, grid, dim3(kThreads), 0, s, p, (const bf16_t*)q_pre, w_q,
                       (const bf16_t*)k_idx, sel, w);
  else
    hipLaunchKernelGGL(sel_dec_score<float>, grid, dim3(kThreads), 0, s, p, (const float*)q_pre, w_q,
                       (const float*)k_idx, sel, w);
  hipLaunchKernelGGL(sel_dec_finish, dim3(p.R * p.batch), dim3(kFT), 0, s, p, top_p, top_k, sel, w);
  return hipGetLastError();
}

int select_decode_max_keys() { return kMaxUnits * kChunk; }

size_t ws_select_blocks(const ProbDev& p) { return align256(sizeof(float2) * (size_t)p.R * blk_slots_per_r(p)); }

hipError_t launch_select_blocks(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                const void* k_idx, const float* top_p, const rtp_selection& sel, void* ws,
                                hipStream_t s) {
  if (p.R == 0) return hipSuccess;
  const int nrows = p.R * p.batch;
  float2* bstat = (float2*)ws;
  dim3 grid(max(1, max_units(p)), nrows);
  if (bf16)
    hipLaunchKernelGGL(sel_blk_score<bf16_t>, grid, dim3(kThreads), 0, s, p, (const bf16_t*)q_pre, w_q,
                       (const bf16_t*)k_idx, sel, bstat);
  else
    hipLaunchKernelGGL(sel_blk_score<float>, grid, dim3(kThreads), 0, s, p, (const float*)q_pre, w_q,
                       (const float*)k_idx, sel, bstat);
  hipLaunchKernelGGL(sel_blk_choose, dim3(nrows), dim3(kThreads), 0, s, p, top_p, sel, (const float2*)bstat);
  return hipGetLastError();
}

}  // namespace rtp
