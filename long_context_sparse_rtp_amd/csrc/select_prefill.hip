// Dynamic top-p for every query row of a prefill, THRESHOLD output.
//
// Definition ("Full Attention Strikes Back ...", paper-graph-ui summary,
// section 3.4 "Dynamic Top-p Selection Mechanism", Eq. 5): over the causal
// prefix n <= pos, softmax of s_n = q_idx . k_idx_n / 4, keys by descending
// score (ties: ascending position), the smallest prefix whose mass reaches p.
// The same kernel with COUNT = true gives the fixed top-k the page ablates
// against (sections "Evaluation Methodology" and "Ablation Studies and
// Robustness Checks"): every token then weighs 1 instead of its mass and the
// target is k instead of p * Z.
// The result of a row is (tau, tie_pos, count): S = {s > tau} U {s == tau,
// n <= tie_pos}; tie_pos = INT_MAX when no token scoring exactly tau is left
// out, so that S = {s >= tau}.  Lists are never materialised (a 128K prefill
// would need ~10^10 entries per head).
//
// A workgroup (4 wave64s) owns 16 query rows of one retrieval head; the rows
// are the 16 columns of the shared MFMA indexer tile and the four waves take
// interleaved 16-key tiles of the causal range.  Scores are never stored:
// each sweep over the keys recomputes them with the same MFMA, so every sweep
// (and the attention kernel) sees identical float32 values.
//
// Per token, with u = (top - s) log2(e) * B the distance below the reference
// top >= max s in units of 1/B octave (B = kBinsPerOctave; top is a
// Cauchy-Schwarz bound, rebased when loose):
//   mass = 2^(31.98 - (top - s) log2 e) as an integer, one FMA and one exp2 of
//          the raw dot product, summed in 64-bit LDS integers (exact and
//          order-independent: the result is deterministic);
//   K    = floor(u * 2^16) clamped to 32 bits (K >> 16 == floor(u)).
// The fixed-point mass of a token is truncated (at most one unit lost), so a
// row's total Z and every cumulative mass carry an error of at most (pos + 1)
// units; the rounding of the exponent's argument (half an ulp of a value below
// 32) and of exp2 add about 8e-7 relative per token.  After the first full
// sweep a row is certified when (pos + 1) <= 2^-17 Z, which keeps a crossing
// within 7.6e-6 + 1.6e-6 of p in cumulative mass (the set tolerance is 1e-5).
// The wide mass is 2^(ms - (top - s) log2 e) with ms = 42 as an exact 64-bit
// integer.  A row whose sampled mean mass (first sweep) is below 2^18 units, or
// whose best sampled key sits 8 octaves or more below the reference, takes it in
// the windowed sweep, together with every other row of that sweep;
// a narrow row that fails the certification repeats the windowed sweep wide; a
// wide row that fails (its mass in a few tokens far above a long tail, with a
// loose reference) takes the full coarse sweep, which lowers its reference to
// within 1/8 octave of the row maximum, where the truncation error is below
// 2^-21 Z for rows up to 2^20 keys.
// A first sweep reads every 8th full tile (and the diagonal tiles) and
// histograms the mass over kNB1 bins of floor(u) (the last one open-ended);
// 16 threads per row scan it for the bin where the cumulative mass reaches p
// times the sampled total (top-k: k times the sampled share of the keys), an
// estimate of the crossing, placed inside its bin by linear interpolation of the
// bin's sampled mass (a top-k target, which needs keys far below the maximum
// too, takes bins wide enough to span the row's score range).  The windowed
// sweep then histograms every key's mass over 254 fine bins centred on that
// estimate (1/256 octave for rows under 64K keys, halving per doubling of the
// row down to 1/4096 octave, so that long rows' crossing bins stay collectable;
// a top-k target's fine bins scale with its sample's bins and widen until the
// window covers three deviations of the sampled rank), plus one bin above and
// one below the window; the scan finds the crossing bin exactly.  A collect sweep
// counts the tokens above the bin's lower edge (taking off the bin's own, which it
// counts as it gathers them) and gathers the bin's tokens; if they are at most kCap, they are sorted by
// (score desc, position asc) (ranks: every candidate against all, 16 threads
// per row) and the crossing token gives tau and tie_pos.  A crossing outside
// the window, a sample with no key within 15 octaves of the reference (the full
// coarse sweep first) or a bin with more than kCap tokens fall back to refinement
// sweeps that histogram
// the mass over the next 8 bits of K inside the chosen range; exact ties too
// large to collect switch the key to the score's bit pattern and then to the
// position (degenerate inputs only).  The refine and collect sweeps compare
// the raw dot product with per-row bounds (exactly the float tests on K) and
// touch LDS only for the few tokens inside the range: a wave tests its whole
// tile first and skips the update code when no lane has a token there.
#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;
constexpr int kNB1 = 256;                       // first-sweep bins
constexpr float kBinsPerOctave = 16.f;          // kNB1 bins span 16 octaves
constexpr int kNB2 = 256;                       // refinement digits (8 bits)
constexpr int kCap = 192;
constexpr float kMaxK = 4294967040.f;           // largest float below 2^32
constexpr int kParts = kThreads / kRows;        // threads per row in the scans

// Sweeps in the order a row can need them; a workgroup runs the lowest phase any
// of its rows is in.
enum { PH_P0 = 0, PH_HIST1 = 1, PH_HISTW = 2, PH_REFINE = 3, PH_COLLECT = 4, PH_DONE = 5 };
constexpr int kFineShift = 12;                  // window bins of short rows: 1/256 octave = 2^12 units of K
// Window bins of a row: 2^fine_shift(pos) units of K.  The number of tokens in the
// crossing bin grows with the row's length, so longer rows take finer bins (down to
// 1/4096 octave above 512K keys) and their crossing bin still fits the candidate buffer.
__device__ __forceinline__ int fine_shift(int pos) {
  return pos < 65536 ? 12 : pos < 131072 ? 11 : pos < 262144 ? 10 : pos < 524288 ? 9 : 8;
}
constexpr int kSample = 8;                      // the first sweep reads every 8th full tile
constexpr int kDepth = 4;                       // full tiles' index keys in flight per wave in a sweep
// Narrow mass scale: a token at the reference weighs 2^31.98 units, so that every
// mass converts to a 32-bit integer (the argument's rounding stays far below 0.02)
constexpr float kNarrowScale = 31.98f;

__device__ __forceinline__ uint32_t desc_key(float s) {
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~u;
}
__device__ __forceinline__ float undesc_key(uint32_t k) {
  const uint32_t a = ~k;
  return __uint_as_float((a & 0x80000000u) ? (a & 0x7FFFFFFFu) : ~a);
}

struct RowCtl {
  double target;
  unsigned long long above;   // fixed-point mass of tokens strictly better than the range
  float top;                  // reference score (>= row max)
  float pval;
  int kval;                   // top-k budget (COUNT)
  uint32_t lo;                // range start in the current key space
  uint32_t kfix, dfix;        // fixed K / desc_key for the tie key spaces
  int sh;                     // digit shift of the range
  int phase, kind;
  int pos;
  int wide;                   // the row's mass is the wide (64-bit) one
  int g0;                     // first fine bin of the window of the windowed sweep
  int fsh;                    // its fine bins are 2^fsh units of K
  int csh;                    // the first sweep's bins are 2^(16 + csh) units of K
  uint32_t cabove;            // tokens strictly better than the range (counted by the collect sweep)
  float tau;
  int tie, count;
};

// Per-lane constants of a row for one sweep.
struct RowK {
  float a20, b20;   // K as float = fma(dot, a20, b20)
  float am, bm;     // mass = 2^fma(dot, am, bm)
  float bw;         // wide mass = 2^fma(dot, am, bw)
  bool wide;
  float lo_f, hi_f; // float range of K for the fast range test
  float dA, dB;     // the same tests on the raw dot: K >= lo <=> d <= dA, K < hi <=> d > dB
  float a12, b12;   // fine bin coordinate (1/256 octave) = fma(dot, a12, b12) = K / 2^12 exactly
  float c12;        // g0 - 1: window bin = clamp(floor(coordinate), c12, c12 + 255) - c12
  int csh;          // the row's first-sweep bin width (RowCtl::csh)
  uint32_t lo;
  int sh, kind, pos;
  uint32_t kfix, dfix;
  bool fast;        // the float range test is exact
};

__device__ __forceinline__ uint32_t key20(float u20) { return (uint32_t)__builtin_amdgcn_fmed3f(u20, 0.f, kMaxK); }

// The largest dot product d with fmaf(d, a, b) >= t, for a < 0 (the map is then
// non-increasing in d, so {d : fmaf(d, a, b) >= t} = {d <= result}): bisection
// over the order-preserving integer image of the floats.  Comparing the raw dot
// with it is exactly the float test on fmaf(d, a, b), one FMA cheaper per pair.
__device__ __forceinline__ float dot_bound(float a, float b, float t) {
  if (t == -INFINITY) return INFINITY;
  if (t == INFINITY) return -INFINITY;
  auto ord = [](float f) { const int i = __float_as_int(f); return (long long)(i ^ ((i >> 31) & 0x7FFFFFFF)); };
  auto unord = [](long long v) { const int i = (int)v; return __int_as_float(i ^ ((i >> 31) & 0x7FFFFFFF)); };
  long long lo = ord(-INFINITY), hi = ord(INFINITY);   // fmaf(-inf, a, b) = +inf >= t; fmaf(+inf, a, b) = -inf < t
  while (hi - lo > 1) {
    const long long mid = lo + (hi - lo) / 2;
    if (fmaf(unord(mid), a, b) >= t) lo = mid; else hi = mid;
  }
  return unord(lo);
}
__device__ __forceinline__ uint32_t mass_narrow(float dot, float am, float bm) {   // < 2^32
  return (uint32_t)__builtin_amdgcn_exp2f(fmaf(dot, am, bm));
}
// The wide mass: the float 2^fma(dot, am, bw) < 2^42 as an exact 64-bit integer
// (its part above 2^32 is hi = floor(f / 2^32); f - hi 2^32 is exact in float).
__device__ __forceinline__ unsigned long long mass_wide(float dot, float am, float bw) {
  const float f = __builtin_amdgcn_exp2f(fmaf(dot, am, bw));
  const uint32_t hi = (uint32_t)(f * 2.3283064365386963e-10f);
  const uint32_t lo = (uint32_t)fmaf((float)hi, -4294967296.f, f);
  return ((unsigned long long)hi << 32) | lo;
}
// Mass scale of a row in wide mode: 2^ws per token at most, so that the 64-bit
// sums of up to 2^(62 - ws) tokens cannot overflow.
__device__ __forceinline__ float wide_scale(int pos) {
  const int nb = 32 - __clz((uint32_t)pos + 1u);   // bits of pos + 1
  return (float)min(42, 62 - nb);
}

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
  const int k0 = key_row0(p, b), L = p.cu_k[b + 1] - p.cu_k[b];
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

// LDS shared by the sweeps (one at a time).
constexpr size_t kHist1Bytes = sizeof(unsigned long long) * kNB1 * kRows;
constexpr size_t kRefineBytes = sizeof(unsigned long long) * kNB2 * kRows;
constexpr size_t kCandBytes = sizeof(unsigned long long) * kRows * kCap;
constexpr size_t kUnionBytes = (kHist1Bytes > kRefineBytes ? (kHist1Bytes > kCandBytes ? kHist1Bytes : kCandBytes)
                                                            : (kRefineBytes > kCandBytes ? kRefineBytes : kCandBytes));
static_assert(kCap <= 256, "the sort's permutation is stored in bytes");
static_assert(kCandBytes + kRows * kCap <= kUnionBytes, "candidates and their permutation share the sweep space");

template <typename T, bool COUNT>
__global__ __launch_bounds__(kThreads, 4) void select_prefill_kernel(
    ProbDev p, const T* __restrict__ q_pre, const float* __restrict__ w_q, const T* __restrict__ k_idx,
    const float* __restrict__ top_p, const int32_t* __restrict__ top_k, rtp_selection sel,
    const uint32_t* __restrict__ kn2) {
  typedef typename IdxFrag<T>::type IF;
  const int tiles_per_b = (p.max_q + kRows - 1) / kRows;
  const int b = blockIdx.x % p.batch;
  const int qt = tiles_per_b - 1 - (int)(blockIdx.x / p.batch);  // longest rows first
  const int r = blockIdx.y;
  const int q0 = p.cu_q[b], Lq = p.cu_q[b + 1] - q0;
  const int k0 = key_row0(p, b), Lk = p.cu_k[b + 1] - p.cu_k[b];
  const int i0 = qt * kRows;
  if (i0 >= Lq) return;
  const int off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile loops run on scalars
  const int col = lane & 15, grp = lane >> 4;

  __shared__ T qidx_s[kRows][kIdxDim];
  __shared__ RowCtl ctl[kRows];
  __shared__ __attribute__((aligned(16))) unsigned char un_s[kUnionBytes];
  __shared__ int ccount_s[kRows];
  __shared__ uint32_t cbetter_s[kRows];
  __shared__ unsigned long long psum_s[kRows][kParts];
  __shared__ int pidx_s[kRows][kParts];
  __shared__ int sweep_s;
  auto h1 = reinterpret_cast<unsigned long long(*)[kRows]>(un_s);                      // [kNB1][kRows]
  auto hm2 = reinterpret_cast<unsigned long long(*)[kRows]>(un_s);                     // [kNB2][kRows]
  unsigned long long* cand = reinterpret_cast<unsigned long long*>(un_s);              // [kRows][kCap]

  // ---- indexer queries of the 16 rows (float64, fixed order, rounded once);
  // rows past the end repeat the last row and are not written back.  The 16
  // pre-RoPE rows and W^Q are staged in LDS (inside the sweep space) first.
  {
    float* wl = reinterpret_cast<float*>(un_s);                     // [16][129] (padded rows)
    T* xl = reinterpret_cast<T*>(wl + kIdxDim * (kHeadDim + 1));    // [16][128]
    for (int e = tid; e < kIdxDim * kHeadDim; e += kThreads) {
      wl[(e >> 7) * (kHeadDim + 1) + (e & 127)] = w_q[(size_t)r * kIdxDim * kHeadDim + e];
      const int row = min(i0 + (e >> 7), Lq - 1);
      xl[e] = q_pre[((size_t)(q0 + row) * p.R + r) * kHeadDim + (e & 127)];
    }
    __syncthreads();
    const int rr = (tid >> 4) & (kRows - 1), j = tid & 15;
    double acc = 0.0;
    for (int d = 0; d < kHeadDim; ++d)
      acc = fma((double)Elem<T>::to_f(xl[rr * kHeadDim + d]), (double)wl[j * (kHeadDim + 1) + d], acc);
    const T qv = Elem<T>::from_d(acc);
    __syncthreads();
    if (tid < kRows * kIdxDim) {
      qidx_s[rr][j] = qv;
      if (i0 + rr < Lq) ((T*)sel.q_idx)[((size_t)r * p.Tq + q0 + i0 + rr) * kIdxDim + j] = qv;
    }
  }
  __syncthreads();
  if (tid < kRows) {
    RowCtl& c = ctl[tid];
    c.pos = off + min(i0 + tid, Lq - 1);
    float qn = 0.f;
#pragma unroll
    for (int j = 0; j < kIdxDim; ++j) {
      const float v = Elem<T>::to_f(qidx_s[tid][j]);
      qn = fmaf(v, v, qn);
    }
    const float kn = __uint_as_float(kn2[r * p.batch + b]);
    c.top = sqrtf(qn * kn) * 0.25f * 1.0009765625f + 1e-30f;
    c.above = 0ull;
    c.cabove = 0u;
    c.lo = 0u; c.sh = 16; c.kind = 0; c.kfix = 0u; c.dfix = 0u;
    c.wide = 0;
    c.tau = -INFINITY; c.tie = 0x7FFFFFFF; c.count = c.pos + 1;
    c.target = 1.0;
    c.g0 = 1;
    c.fsh = kFineShift;
    // A count target needs the keys far below the maximum too (a mass target does not:
    // they weigh nothing), so the first sweep's 256 bins must span the row's score range,
    // at most 2 top log2(e) octaves: bins of 1/16 octave cover 16, and a wide range takes
    // bins 2^csh times as wide (up to half the range may fall in the last, open bin).
    c.csh = 0;
    if (COUNT) {
      const float range = 2.f * c.top * kLog2e;
      while (c.csh < 8 && range > 32.f * (float)(1 << c.csh)) ++c.csh;
    }
    if (COUNT) {
      c.pval = 0.f;
      c.kval = max(top_k[b], 1);
      c.phase = (c.kval <= c.pos) ? PH_P0 : PH_DONE;      // k >= pos + 1: every key
    } else {
      c.pval = top_p[b];
      c.kval = 0;
      c.phase = (c.pval < 1.f) ? PH_P0 : PH_DONE;        // p >= 1 (or NaN): every key
    }
  }
  __syncthreads();

  IF qxf;
  load_idx_frag(qxf, &qidx_s[col][4 * grp]);
  const T* kxb = k_idx + ((size_t)r * p.Tk + k0) * kIdxDim;
  const int p0 = off + i0;                           // smallest position of the 16 rows
  const int pos_hi = off + min(i0 + kRows, Lq) - 1;
  const int ntile = pos_hi / 16 + 1;
  const int nfull = p0 / 16;                         // tiles entirely below every row's position

  auto tile_dot = [&](int t) -> f32x4 {
    IF kxf;
    const int key = 16 * t + col;
    if (key < Lk) {
      load_idx_frag(kxf, kxb + (size_t)key * kIdxDim + 4 * grp);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) kxf.v[j] = 0;
    }
    return idx_dot_tile(kxf, qxf);
  };
  // byte offsets from the row block's first index key: a scalar base plus one
  // 32-bit lane offset (the keys of one retrieval head span well under 4 GB)
  const char* kxc = reinterpret_cast<const char*>(kxb);
  const uint32_t lane_off = (uint32_t)(col * kIdxDim + 4 * grp) * (uint32_t)sizeof(T);
  auto load_full = [&](IF& f, int t) {
    const uint32_t tt = (uint32_t)__builtin_amdgcn_readfirstlane(min(t, nfull - 1));
    load_idx_frag(f, reinterpret_cast<const T*>(kxc + (tt * (16u * kIdxDim * (uint32_t)sizeof(T)) + lane_off)));
  };
  // Full tiles t, t + stride, ... (every key exists and lies below every row's
  // position) in groups of D with D tiles' index keys in flight: each register set
  // is reloaded with the tile D strides ahead as soon as its product is issued
  // (unconditional loads: past the last full tile they re-read it).  A sweep is
  // bound by the latency of these loads, not by its arithmetic, unless several
  // are in flight.  Returns the first tile of the wave not visited.
  auto sweep_full = [&](auto depth, int t, int stride, auto&& body) -> int {
    constexpr int D = decltype(depth)::value;
    if (t + (D - 1) * stride < nfull) {
      IF f[D];
#pragma unroll
      for (int j = 0; j < D; ++j) load_full(f[j], t + j * stride);
      do {
#pragma unroll
        for (int j = 0; j < D; ++j) {
          const f32x4 d = idx_dot_tile(f[j], qxf);
          load_full(f[j], t + (D + j) * stride);
          body(d, t + j * stride, false);
        }
        t += D * stride;
      } while (t + (D - 1) * stride < nfull);
    }
    return t;
  };
  // every tile of the wave: the full tiles kDepth, then two, in flight, then the
  // rest (the diagonal tiles, bounds-checked) one at a time
  auto sweep_tiles = [&](auto&& body) {
    int t = sweep_full(std::integral_constant<int, kDepth>{}, w, kWaves, body);
    t = sweep_full(std::integral_constant<int, 2>{}, t, kWaves, body);
    for (; t < ntile; t += kWaves) body(tile_dot(t), t, t >= nfull);
  };
  // every kSample-th full tile (same prefetch scheme), then every diagonal tile
  auto sweep_sample = [&](auto&& body) {
    constexpr int kStride = kSample * kWaves;
    int t = sweep_full(std::integral_constant<int, kDepth>{}, kSample * w, kStride, body);
    for (; t < nfull; t += kStride) body(tile_dot(t), t, false);
    for (int td = nfull + w; td < ntile; td += kWaves) body(tile_dot(td), td, true);
  };

  // thread (row, part) of the parallel scans
  const int srow = tid / kParts, spart = tid % kParts;

  for (int iter = 0; iter < 64; ++iter) {
    if (tid == 0) {
      int k = PH_DONE;
      for (int rr = 0; rr < kRows; ++rr) k = min(k, ctl[rr].phase);
      sweep_s = k;
      // a windowed sweep is narrow or wide for all its rows: one wide row makes all wide
      // (the wide mass is the more precise one; a row's later sweeps follow its mode)
      if (k == PH_HISTW) {
        bool anyw = false;
        for (int rr = 0; rr < kRows; ++rr) anyw |= (ctl[rr].phase == PH_HISTW) && (ctl[rr].wide != 0);
        if (anyw)
          for (int rr = 0; rr < kRows; ++rr)
            if (ctl[rr].phase == PH_HISTW) ctl[rr].wide = 1;
      }
    }
    __syncthreads();
    const int sweep = sweep_s;
    if (sweep == PH_DONE) break;
    // per-lane constants of this lane's row
    RowK rk;
    {
      const RowCtl& c = ctl[col];
      const bool active = c.phase == sweep;
      rk.a20 = -kLog2e * 0.25f * kBinsPerOctave * 65536.f;
      rk.b20 = c.top * kLog2e * kBinsPerOctave * 65536.f;
      rk.am = kLog2e * 0.25f;
      rk.bm = kNarrowScale - c.top * kLog2e;
      rk.bw = wide_scale(c.pos) - c.top * kLog2e;
      rk.wide = c.wide != 0;
      rk.lo = c.lo;
      rk.sh = c.sh;
      rk.kind = c.kind;
      rk.kfix = c.kfix;
      rk.dfix = c.dfix;
      rk.pos = active ? c.pos : -1;
      const int width = (sweep == PH_REFINE) ? c.sh + 8 : c.sh;
      // the float test of K's range is exact when both ends are exact floats
      const double hi = (double)c.lo + (double)(1ull << min(width, 32));
      const bool lo_exact = (double)(float)c.lo == (double)c.lo;
      const bool hi_exact = hi >= 4294967040.0 || (double)(float)hi == hi;
      rk.fast = (c.kind == 0) && lo_exact && hi_exact;
      rk.lo_f = (c.lo == 0u) ? -INFINITY : (float)c.lo;
      rk.hi_f = (hi >= 4294967040.0) ? INFINITY : (float)hi;
      rk.dA = dot_bound(rk.a20, rk.b20, rk.lo_f);
      rk.dB = dot_bound(rk.a20, rk.b20, rk.hi_f);
      rk.a12 = ldexpf(rk.a20, -c.fsh);   // power-of-two scalings: exact
      rk.b12 = ldexpf(rk.b20, -c.fsh);
      rk.c12 = (float)(c.g0 - 1);
      rk.csh = c.csh;
    }
    {
      uint32_t* z = reinterpret_cast<uint32_t*>(un_s);
      const int nz = (int)(((sweep == PH_P0 || sweep == PH_HIST1 || sweep == PH_HISTW) ? kHist1Bytes
                            : (sweep == PH_REFINE) ? kRefineBytes : 0) / 4);
      for (int e = tid; e < nz; e += kThreads) z[e] = 0u;
    }
    if (tid < kRows) { ccount_s[tid] = 0; cbetter_s[tid] = 0u; }
    __syncthreads();

    const bool all_fast = __builtin_amdgcn_ballot_w64(!rk.fast) == 0;
    // coarse bin coordinate K / 2^16 (exact power-of-two scaling); the first sweep's bins
    // are 2^csh times wider for rows whose count target needs a wide score range
    const int cs = 16 + ((sweep == PH_P0) ? rk.csh : 0);
    const float a1 = ldexpf(rk.a20, -cs), b1 = ldexpf(rk.b20, -cs);
    uint32_t better = 0u;

    // coarse histogram: bins of 1/16 octave below the reference, the last open-ended
    auto hist_coarse = [&](const f32x4& d, int t, bool check) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * t + 4 * grp + i;
        if (check && n > rk.pos) continue;
        const float u = fmaf(d[i], a1, b1);
        const uint32_t bin = (uint32_t)__builtin_amdgcn_fmed3f(u, 0.f, (float)(kNB1 - 1));
        atomicAdd(&h1[bin][col], COUNT ? 1ull : (unsigned long long)mass_narrow(d[i], rk.am, rk.bm));
      }
    };
    // the same with the wide mass for rows that need it (the full coarse sweep only)
    auto hist_coarse_w = [&](const f32x4& d, int t, bool check) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = 16 * t + 4 * grp + i;
        if (check && n > rk.pos) continue;
        const float u = fmaf(d[i], a1, b1);
        const uint32_t bin = (uint32_t)__builtin_amdgcn_fmed3f(u, 0.f, (float)(kNB1 - 1));
        atomicAdd(&h1[bin][col], COUNT ? 1ull : rk.wide ? mass_wide(d[i], rk.am, rk.bw)
                                                        : (unsigned long long)mass_narrow(d[i], rk.am, rk.bm));
      }
    };
    // wide rows among the rows this sweep serves (rk.pos < 0 marks a row in another phase)
    const bool any_wide = __builtin_amdgcn_ballot_w64(rk.wide && rk.pos >= 0) != 0;
    if (sweep == PH_P0) {
      sweep_sample(hist_coarse);
    } else if (sweep == PH_HIST1) {
      if (any_wide) sweep_tiles(hist_coarse_w); else sweep_tiles(hist_coarse);
    } else if (sweep == PH_HISTW) {
      // window of 254 bins of 1/256 octave; bin 0 holds everything above it, bin 255 everything below.
      // The coordinate is K / 2^12 exactly (a power-of-two scaling of the key's FMA) and
      // subtracting the integer c12 from it is exact, so bin j holds K in [(g0+j-1) << 12, (g0+j) << 12).
      static_assert(kRows * sizeof(unsigned long long) == 128, "a window bin row is 128 bytes");
      // floor(coordinate) clamped to [c12, c12 + 255] is c12 + the bin, so the lane's
      // LDS base absorbs -c12 and the bin costs a clamp, a conversion and a shift-add
      const float c12hi = rk.c12 + 255.f;
      char* hbase = reinterpret_cast<char*>(&h1[0][col]) - (ptrdiff_t)(int)rk.c12 * (kRows * 8);
      if (!any_wide) {
        sweep_tiles([&](const f32x4& d, int t, bool check) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = 16 * t + 4 * grp + i;
            if (check && n > rk.pos) continue;
            const float u12 = fmaf(d[i], rk.a12, rk.b12);
            const uint32_t gb = (uint32_t)__builtin_amdgcn_fmed3f(u12, rk.c12, c12hi);
            atomicAdd(reinterpret_cast<unsigned long long*>(hbase + (gb << 7)),
                      COUNT ? 1ull : (unsigned long long)mass_narrow(d[i], rk.am, rk.bm));
          }
        });
      } else {   // every row in this sweep takes the wide mass (see the phase choice)
        sweep_tiles([&](const f32x4& d, int t, bool check) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = 16 * t + 4 * grp + i;
            if (check && n > rk.pos) continue;
            const float u12 = fmaf(d[i], rk.a12, rk.b12);
            const uint32_t gb = (uint32_t)__builtin_amdgcn_fmed3f(u12, rk.c12, c12hi);
            atomicAdd(reinterpret_cast<unsigned long long*>(hbase + (gb << 7)),
                      COUNT ? 1ull : mass_wide(d[i], rk.am, rk.bw));
          }
        });
      }
    } else if (sweep == PH_REFINE && all_fast) {
      sweep_tiles([&](const f32x4& d, int t, bool check) {
        bool inr[4];
        bool any = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = 16 * t + 4 * grp + i;
          const bool valid = !check || n <= rk.pos;
          inr[i] = valid && d[i] <= rk.dA && d[i] > rk.dB;
          any |= inr[i];
        }
        if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (inr[i]) {
              const uint32_t dig = (key20(fmaf(d[i], rk.a20, rk.b20)) - rk.lo) >> rk.sh;
              atomicAdd(&hm2[dig][col], COUNT ? 1ull : rk.wide ? mass_wide(d[i], rk.am, rk.bw)
                                                               : (unsigned long long)mass_narrow(d[i], rk.am, rk.bm));
            }
          }
        }
      });
    } else if (sweep == PH_COLLECT && all_fast) {
      sweep_tiles([&](const f32x4& d, int t, bool check) {
        bool inr[4];
        bool any = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = 16 * t + 4 * grp + i;
          const bool valid = !check || n <= rk.pos;
          // counted: every token above the range's lower edge (the range's own tokens,
          // which ccount counts, are taken off after the sweep); scores are finite
          const bool gtb = valid && d[i] > rk.dB;
          better += gtb ? 1u : 0u;
          inr[i] = gtb && d[i] <= rk.dA;
          any |= inr[i];
        }
        if (__builtin_amdgcn_ballot_w64(any)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (inr[i]) {
              const int n = 16 * t + 4 * grp + i;
              const int slot = atomicAdd(&ccount_s[col], 1);
              if (slot < kCap)
                cand[col * kCap + slot] = ((unsigned long long)desc_key(idx_score(d[i])) << 32) | (uint32_t)n;
            }
          }
        }
      });
    } else {
      // general path: integer keys and the tie key spaces
      sweep_tiles([&](const f32x4& d, int t, bool) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int n = 16 * t + 4 * grp + i;
          if (n > rk.pos) continue;
          const float u20 = fmaf(d[i], rk.a20, rk.b20);
          const uint32_t K = key20(u20);
          const float s = idx_score(d[i]);
          uint32_t key = K;
          bool ok = true;
          bool bt;
          if (rk.kind >= 1) {
            const uint32_t dk = desc_key(s);
            ok = (K == rk.kfix);
            if (rk.kind == 1) {
              key = dk;
              bt = (K < rk.kfix) || (K == rk.kfix && dk < rk.lo);
            } else {
              ok = ok && (dk == rk.dfix);
              key = (uint32_t)n;
              bt = (K < rk.kfix) || (K == rk.kfix && (dk < rk.dfix || (dk == rk.dfix && (uint32_t)n < rk.lo)));
            }
          } else {
            bt = K < rk.lo;
          }
          const int width = (sweep == PH_REFINE) ? rk.sh + 8 : rk.sh;
          const uint32_t dk2 = key - rk.lo;
          const bool inr = ok && ((width >= 32) ? (key >= rk.lo) : ((dk2 >> width) == 0u));
          if (sweep == PH_COLLECT) better += bt ? 1u : 0u;
          if (!inr) continue;
          if (sweep == PH_REFINE) {
            const uint32_t dig = dk2 >> rk.sh;
            atomicAdd(&hm2[dig][col], COUNT ? 1ull : rk.wide ? mass_wide(d[i], rk.am, rk.bw)
                                                             : (unsigned long long)mass_narrow(d[i], rk.am, rk.bm));
          } else {
            const int slot = atomicAdd(&ccount_s[col], 1);
            if (slot < kCap) cand[col * kCap + slot] = ((unsigned long long)desc_key(s) << 32) | (uint32_t)n;
          }
        }
      });
    }
    if (sweep == PH_COLLECT) {
      better += __shfl_xor(better, 16);
      better += __shfl_xor(better, 32);
      if (grp == 0) atomicAdd(&cbetter_s[col], better);
    }
    __syncthreads();
    if (sweep == PH_COLLECT && all_fast) {   // the fast collect counted the range's tokens too
      if (tid < kRows) cbetter_s[tid] -= (uint32_t)ccount_s[tid];
      __syncthreads();
    }

    // ---- per-row controller.  The histogram scans run on 16 threads per row:
    // part sums, then the part holding the crossing walks its bins.
    const bool act = ctl[srow].phase == sweep;
    if (sweep == PH_P0) {
      // estimate the crossing from the sample; the windowed sweep then bins finely
      // around it.  A loose reference (best sampled key 8 to 15 octaves below it)
      // takes the wide mass there; a sample with nothing above the last 16 bins, or
      // a crossing the scan does not find, takes the full coarse sweep instead.
      constexpr int PB = kNB1 / kParts;
      unsigned long long sp = 0ull;
      int first = kNB1;
      if (act) {
        for (int j = 0; j < PB; ++j) {
          const unsigned long long hv = h1[spart * PB + j][srow];
          if (first == kNB1 && hv != 0ull) first = spart * PB + j;
          sp += hv;
        }
      }
      psum_s[srow][spart] = sp;
      pidx_s[srow][spart] = first;
      __syncthreads();
      if (act && spart == 0) ctl[srow].phase = PH_HIST1;   // default: the full coarse sweep
      __syncthreads();
      if (act) {
        RowCtl& rc = ctl[srow];
        unsigned long long Z = 0ull, pre = 0ull;
        int blo = kNB1;
        for (int q = 0; q < kParts; ++q) {
          if (q < spart) pre += psum_s[srow][q];
          Z += psum_s[srow][q];
          blo = min(blo, pidx_s[srow][q]);
        }
        if (blo < kNB1 - 16 && Z != 0ull) {
          // the sample holds a share Z / (pos + 1) of the keys: scale a count target by it
          const double target = COUNT ? fmax((double)rc.kval * (double)Z / (double)(rc.pos + 1), 1.0)
                                      : fmax((double)rc.pval * (double)Z, 1.0);
          if ((double)pre < target && target <= (double)(pre + sp)) {
            unsigned long long cm = pre;
            int bstar = spart * PB + PB - 1;
            for (int j = 0; j < PB; ++j) {
              const unsigned long long hv = h1[spart * PB + j][srow];
              if ((double)(cm + hv) >= target) { bstar = spart * PB + j; break; }
              cm += hv;
            }
            // window of 254 fine bins centred on the estimate: the target's place inside
            // the coarse bin by linear interpolation of the bin's sampled mass.  The fine
            // bins keep their share of a coarse bin when the coarse bins are wider.
            const int cw = 16 + rc.csh;                               // coarse bin: 2^cw units of K
            int fsh = fine_shift(rc.pos) + rc.csh;
            const unsigned long long hb = h1[bstar][srow];
            const double fr = (hb != 0ull) ? fmin(fmax((target - (double)cm) / (double)hb, 0.0), 1.0) : 0.5;
            long long centre = ((long long)bstar << cw) + (long long)(fr * (double)(1ll << cw));
            if (COUNT) {
              // A count target's sampled rank is off by about sqrt(target) keys; where the
              // sample is sparse (a thin tail of high scores) that spans many coarse bins.
              // The window then takes wider bins so that it covers the coarse bins where
              // the sampled count is within three deviations of the target.
              const double dev = 3.0 * sqrt(target) + 1.0;
              int b1 = bstar;
              unsigned long long c1 = cm;                                   // count above b1
              while (b1 > 0 && (double)c1 >= target - dev) { --b1; c1 -= h1[b1][srow]; }
              int b2 = bstar;
              unsigned long long c2 = cm + hb;                              // count down to b2
              while (b2 < kNB1 - 2 && (double)c2 < target + dev) { ++b2; c2 += h1[b2][srow]; }
              const long long span = (long long)(b2 - b1 + 1) << cw;
              if ((254ll << fsh) < span) {
                while (fsh < 24 && (254ll << fsh) < span) ++fsh;
                centre = ((long long)b1 << cw) + span / 2;
              }
            }
            rc.fsh = fsh;
            // (the window's last bin must end inside the 32-bit key: (g0 + 254) << fsh < 2^32)
            rc.g0 = max(1, min((int)(centre >> fsh) - 127, (int)(0xFFFFFFFFu >> fsh) - 254));
            rc.phase = PH_HISTW;
            // a sample whose mean mass is below 2^18 units predicts a row that would fail
            // the certification after the windowed sweep: it takes the wide mass there
            // directly.  The sample holds every 8th full tile and the diagonal tiles.
            const double nsamp = 16.0 * (double)((nfull + kSample - 1) / kSample) + (double)(rc.pos + 1 - 16 * nfull);
            if (!COUNT && ((double)Z < nsamp * 262144.0 || blo >= kNB1 / 2)) rc.wide = 1;
          }
        }
      }
    } else if (sweep == PH_HISTW) {
      constexpr int PB = kNB1 / kParts;
      unsigned long long sp = 0ull;
      if (act) {
        for (int j = 0; j < PB; ++j) sp += h1[spart * PB + j][srow];
      }
      psum_s[srow][spart] = sp;
      __syncthreads();
      if (act && spart == 0) ctl[srow].phase = PH_HIST1;   // default (the scan below always claims)
      __syncthreads();
      if (act) {
        RowCtl& rc = ctl[srow];
        unsigned long long Z = 0ull, pre = 0ull;
        for (int q = 0; q < kParts; ++q) {
          if (q < spart) pre += psum_s[srow][q];
          Z += psum_s[srow][q];
        }
        const double target = COUNT ? (double)rc.kval : fmax((double)rc.pval * (double)Z, 1.0);
        // certification: the truncation error of Z (at most one unit per key) must stay
        // below 2^-17 Z; otherwise the row restarts from the coarse sweep with the wide mass
        const bool certified = COUNT || (double)(rc.pos + 1) * 131072.0 <= (double)Z;
        if (!certified) {
          // narrow: the windowed sweep again with the wide mass (its window still holds);
          // already wide: the full coarse sweep, which also tightens the reference
          if (spart == 0 && !rc.wide) {
            rc.wide = 1;
            rc.phase = PH_HISTW;
          }
        } else if ((double)pre < target && target <= (double)(pre + sp)) {
          unsigned long long cm = pre;
          int jstar = spart * PB + PB - 1;
          for (int j = 0; j < PB; ++j) {
            const unsigned long long hv = h1[spart * PB + j][srow];
            if ((double)(cm + hv) >= target) { jstar = spart * PB + j; break; }
            cm += hv;
          }
          rc.target = target;
          rc.above = cm;
          const int g0 = rc.g0;
          if (jstar >= 1 && jstar <= 254) {        // inside the window: gather the bin's keys
            rc.lo = (uint32_t)(g0 + jstar - 1) << rc.fsh;
            rc.sh = rc.fsh;
            rc.phase = PH_COLLECT;
          } else if (jstar == 0) {                 // above the window: refine [0, g0 << 12)
            const uint32_t span = ((uint32_t)g0 << rc.fsh) - 1u;
            const int wdt = 32 - __clz(span);
            rc.lo = 0u;
            rc.sh = max(wdt, 8) - 8;
            rc.phase = PH_REFINE;
          } else {                                 // below the window: refine the rest
            rc.lo = (uint32_t)(g0 + 254) << rc.fsh;
            rc.sh = 24;
            rc.phase = PH_REFINE;
          }
        }
      }
    } else if (sweep == PH_HIST1) {
      constexpr int PB = kNB1 / kParts;
      unsigned long long sp = 0ull;
      int first = kNB1;
      if (act) {
        for (int j = 0; j < PB; ++j) {
          const unsigned long long hv = h1[spart * PB + j][srow];
          if (first == kNB1 && hv != 0ull) first = spart * PB + j;
          sp += hv;
        }
      }
      psum_s[srow][spart] = sp;
      pidx_s[srow][spart] = first;
      __syncthreads();
      if (act) {
        RowCtl& rc = ctl[srow];
        unsigned long long Z = 0ull, pre = 0ull;
        int blo = kNB1;
        for (int q = 0; q < kParts; ++q) {
          if (q < spart) pre += psum_s[srow][q];
          Z += psum_s[srow][q];
          blo = min(blo, pidx_s[srow][q]);
        }
        // a narrow row whose truncation error bound fails the certification
        // (see the PH_HISTW controller) switches to the wide mass and sweeps again
        const bool uncertified = !COUNT && !rc.wide && (double)(rc.pos + 1) * 131072.0 > (double)Z;
        if (blo >= kNB1 / 2 || Z == 0ull || (rc.wide && blo > 2)) {
          // loose bound (the best token sits >= 8 octaves below it; for a wide row, more
          // than 1/8 octave): lower the reference to just above the best token and
          // histogram again
          if (spart == 0) {
            const int bl = (blo >= kNB1) ? kNB1 - 1 : blo;
            rc.top = rc.top - (float)(bl - 1) / (kBinsPerOctave * kLog2e);
          }
        } else if (uncertified) {
          if (spart == 0) rc.wide = 1;
        } else {
          const double target = COUNT ? (double)rc.kval : fmax((double)rc.pval * (double)Z, 1.0);
          if ((double)pre < target && target <= (double)(pre + sp)) {
            unsigned long long cm = pre;
            int bstar = spart * PB + PB - 1;
            for (int j = 0; j < PB; ++j) {
              const unsigned long long hv = h1[spart * PB + j][srow];
              if ((double)(cm + hv) >= target) { bstar = spart * PB + j; break; }
              cm += hv;
            }
            rc.target = target;
            rc.above = cm;
            rc.lo = (uint32_t)bstar << 16;
            rc.sh = (bstar < kNB1 - 1) ? 8 : 24;   // the last bin spans the rest of the 32-bit key
            rc.phase = PH_REFINE;
          }
        }
      }
    } else if (sweep == PH_REFINE) {
      constexpr int PD = kNB2 / kParts;
      unsigned long long sp = 0ull;
      int lastne = -1;
      if (act) {
        for (int j = 0; j < PD; ++j) {
          const unsigned long long hv = hm2[spart * PD + j][srow];
          sp += hv;
          if (hv != 0ull) lastne = spart * PD + j;
        }
      }
      psum_s[srow][spart] = sp;
      pidx_s[srow][spart] = lastne;
      __syncthreads();
      // read the row state and the part sums, then (after a barrier every thread
      // reaches) the part holding the crossing digit updates the row
      bool mine = false, crosses = true;
      unsigned long long pre = 0ull;
      int last = -1;
      double target = 0.0;
      if (act) {
        const RowCtl& rc = ctl[srow];
        pre = rc.above;
        unsigned long long tot = rc.above;
        for (int q = 0; q < kParts; ++q) {
          if (q < spart) pre += psum_s[srow][q];
          tot += psum_s[srow][q];
          last = max(last, pidx_s[srow][q]);
        }
        target = rc.target;
        // the part holding the crossing digit; if rounding left the target just beyond
        // the range, the part holding the last digit with mass
        crosses = (double)tot >= target;
        mine = crosses ? ((double)pre < target && target <= (double)(pre + sp))
                       : (last < 0 ? spart == 0 : (last >= spart * PD && last < spart * PD + PD));
      }
      __syncthreads();
      if (mine) {
        RowCtl& rc = ctl[srow];
        unsigned long long cm = pre;
        int dstar = crosses ? spart * PD + PD - 1 : max(last, 0);
        if (crosses) {
          for (int j = 0; j < PD; ++j) {
            const int dg = spart * PD + j;
            const unsigned long long hv = hm2[dg][srow];
            if ((double)(cm + hv) >= target) { dstar = dg; break; }
            cm += hv;
          }
        } else {
          for (int dg = spart * PD; dg < dstar; ++dg) cm += hm2[dg][srow];
        }
        rc.above = cm;
        rc.lo = rc.lo + ((uint32_t)dstar << rc.sh);
        rc.phase = PH_COLLECT;
      }
    } else if (sweep == PH_COLLECT) {
      const int ncr = act ? ccount_s[srow] : 0;
      const bool over = ncr > kCap;
      if (over && spart == 0) {
        // too many tokens in the range: refine it further
        RowCtl& rc = ctl[srow];
        if (rc.sh >= 8) {
          rc.sh -= 8;
        } else if (rc.sh > 0) {
          rc.sh = 0;   // a narrower range: refine to single key values first (the digits cover a superset)
        } else if (rc.kind == 0) {
          rc.kind = 1; rc.kfix = rc.lo; rc.lo = 0u; rc.sh = 24;
        } else {
          rc.kind = 2; rc.dfix = rc.lo; rc.lo = 0u; rc.sh = 23;
        }
        rc.phase = PH_REFINE;
      }
      // Sort the candidates by (desc_key, position), both ascending, with ranks: the
      // keys are distinct, so a candidate's rank is the number of smaller ones.  Each
      // of the row's 16 threads ranks kCap / 16 of them against all, a few at a time,
      // and records the permutation (candidate index by rank) in LDS.
      constexpr int E = kCap / kParts;
      constexpr int EC = 4;
      const int nc = over ? 0 : ncr;
      const unsigned long long* cd = cand + srow * kCap;
      unsigned char* perm = un_s + kCandBytes + srow * kCap;
#pragma unroll 1
      for (int c0 = 0; c0 < E; c0 += EC) {
        if (spart + c0 * kParts >= nc) break;
        unsigned long long xv[EC];
        int rank[EC];
#pragma unroll
        for (int e = 0; e < EC; ++e) {
          const int a = spart + (c0 + e) * kParts;
          xv[e] = (a < nc) ? cd[a] : ~0ull;
          rank[e] = 0;
        }
        for (int jj = 0; jj < nc; ++jj) {
          const unsigned long long v = cd[jj];
#pragma unroll
          for (int e = 0; e < EC; ++e) rank[e] += (v < xv[e]) ? 1 : 0;
        }
#pragma unroll
        for (int e = 0; e < EC; ++e) {
          const int a = spart + (c0 + e) * kParts;
          if (a < nc) perm[rank[e]] = (unsigned char)a;
        }
      }
      __syncthreads();
      // The crossing in sorted order: the first candidate at which the mass above
      // the range plus the candidates' cumulative mass reaches the target (the last
      // candidate if none does).  Thread q sums ranks [q E, q E + E); the part where
      // the cumulative mass crosses walks its ranks.
      const float am = kLog2e * 0.25f, bm = kNarrowScale - ctl[srow].top * kLog2e;
      const float bw = wide_scale(ctl[srow].pos) - ctl[srow].top * kLog2e;
      const bool rwide = ctl[srow].wide != 0;
      auto cmass = [&](int k) -> unsigned long long {
        if (COUNT) return 1ull;
        const float dk = undesc_key((uint32_t)(cd[perm[k]] >> 32)) * 4.f;
        return rwide ? mass_wide(dk, am, bw) : (unsigned long long)mass_narrow(dk, am, bm);
      };
      const int a0 = spart * E;
      unsigned long long sp = 0ull;
      for (int k = a0; k < min(a0 + E, nc); ++k) sp += cmass(k);
      psum_s[srow][spart] = sp;
      __syncthreads();
      if (act && !over) {
        RowCtl& rc = ctl[srow];
        unsigned long long pre = rc.above, tot = rc.above;
        for (int q = 0; q < kParts; ++q) {
          if (q < spart) pre += psum_s[srow][q];
          tot += psum_s[srow][q];
        }
        const double target = rc.target;
        const bool crosses = (double)tot >= target;
        const bool mine = nc > 0 && (crosses ? ((spart == 0 && (double)pre >= target) ||
                                                ((double)pre < target && target <= (double)(pre + sp)))
                                             : (a0 <= nc - 1 && nc - 1 < a0 + E));
        if (mine) {
          int js = min(a0 + E, nc) - 1;
          unsigned long long cm = pre;
          for (int k = a0; k < min(a0 + E, nc); ++k) {
            const unsigned long long m = cmass(k);
            if ((double)(cm + m) >= target) { js = k; break; }
            cm += m;
          }
          const unsigned long long xs = cd[perm[js]];
          rc.tau = undesc_key((uint32_t)(xs >> 32));
          rc.tie = (int)(uint32_t)(xs & 0xFFFFFFFFull);
          rc.count = (int)cbetter_s[srow] + js + 1;
          // every token scoring exactly tau is a candidate unless the position key was needed;
          // if none of them is left out, the set is simply {s >= tau}
          const bool excluded = (js + 1 < nc) && ((uint32_t)(cd[perm[js + 1]] >> 32) == (uint32_t)(xs >> 32));
          if (rc.kind < 2 && !excluded) rc.tie = 0x7FFFFFFF;
        }
        if (spart == 0) {
          rc.cabove = cbetter_s[srow];
          rc.phase = PH_DONE;
        }
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
                                 const void* k_idx, const float* top_p, const int32_t* top_k,
                                 const rtp_selection& sel, void* ws, hipStream_t s) {
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
  if (bf16 && top_k)
    hipLaunchKernelGGL((select_prefill_kernel<bf16_t, true>), grid, dim3(kThreads), 0, s, p, (const bf16_t*)q_pre,
                       w_q, (const bf16_t*)k_idx, top_p, top_k, sel, (const uint32_t*)kn2);
  else if (bf16)
    hipLaunchKernelGGL((select_prefill_kernel<bf16_t, false>), grid, dim3(kThreads), 0, s, p, (const bf16_t*)q_pre,
                       w_q, (const bf16_t*)k_idx, top_p, top_k, sel, (const uint32_t*)kn2);
  else if (top_k)
    hipLaunchKernelGGL((select_prefill_kernel<float, true>), grid, dim3(kThreads), 0, s, p, (const float*)q_pre,
                       w_q, (const float*)k_idx, top_p, top_k, sel, (const uint32_t*)kn2);
  else
    hipLaunchKernelGGL((select_prefill_kernel<float, false>), grid, dim3(kThreads), 0, s, p, (const float*)q_pre,
                       w_q, (const float*)k_idx, top_p, top_k, sel, (const uint32_t*)kn2);
  return hipGetLastError();
}

}  // namespace rtp
