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
//   - a row is (retrieval slot, sequence), or (tile of local heads of one KV
//     group, sequence); tiles hold one head at present: holding several lets
//     a K/V row feed all of them, but costs more in cross-lane reductions;
//   - every row's key set is cut into equal splits of at most 1024 entries,
//     sized from the total entry count so that the splits of all rows fit the
//     resident grid once; the splits form one flat work list (prefix sums of the
//     per-row split counts, computed by every workgroup) that the grid walks
//     round-robin, so ragged rows and sparse sets leave no idle workgroups;
//   - a split's key positions are staged in LDS with one coalesced read, so
//     the K/V gathers never wait on the list;
//   - 16 lanes share a token, each lane holding 8 of the 128 dims, so one K
//     row and one V row are single coalesced 256-byte (bf16) segments; each
//     16-lane group keeps two batches of 4 tokens in flight (the next batch
//     is requested before the current one is used);
//   - each group keeps an online-softmax state (max, sum, 8 accumulators) per
//     head in registers; groups merge through LDS, splits merge in a second
//     kernel by log-sum-exp.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int kThreads = 256;
constexpr int kSplit = 1024;             // most entries per split
constexpr int kMinSplit = 64;            // fewest entries per split (unless a row holds fewer)
constexpr int kBalance = 1;              // 1: size splits so that every row fits the grid once; 0: kSplit
constexpr int kGroups = kThreads / 16;   // 16-lane groups per workgroup
constexpr int kUnroll = 4;               // tokens per group per batch
constexpr int kStep = kGroups * kUnroll; // tokens per workgroup per batch
constexpr int kPart = kHeadDim + 2;      // partial record: m, l, o[128]
constexpr int kWgPerCu = 4;              // resident workgroups per CU (VGPR-bound)
constexpr int kMaxRowsLds = 8192;        // rows per call + 1 (the split prefix lives in LDS)
constexpr int kMaxTileHeads = 1;         // local heads per row (one: the tile form costs more in cross-lane
                                         // reductions than it saves in L2 reads)

struct RowInfo {
  int b, qrow, k0, L, count, g, nh;
  int hfirst;   // mode 0: the query head; mode 1: index of the tile's first local head
};

__device__ __forceinline__ RowInfo row_info(const ProbDev& p, int mode, int row, const rtp_selection& sel) {
  RowInfo ri;
  ri.b = row % p.batch;
  const int hi = row / p.batch;
  ri.k0 = key_row0(p, ri.b);
  ri.L = p.cu_k[ri.b + 1] - p.cu_k[ri.b];
  ri.qrow = p.cu_q[ri.b];
  if (mode == 0) {
    ri.hfirst = p.ret_heads[hi];
    ri.nh = 1;
    ri.g = kv_of(p, ri.hfirst);
    ri.count = sel.count[(size_t)hi * p.Tq + ri.qrow];
  } else {
    ri.hfirst = p.ltile_start[hi];
    ri.nh = p.ltile_cnt[hi];
    ri.g = kv_of(p, p.local_heads[ri.hfirst]);
    const int W = min(p.window, ri.L);
    const int ns = min(p.n_sink, ri.L - W);
    ri.count = ns + W;
  }
  return ri;
}
__device__ __forceinline__ int head_of(const ProbDev& p, int mode, const RowInfo& ri, int i) {
  return (mode == 0) ? ri.hfirst : p.local_heads[ri.hfirst + i];
}

// j-th key position of a local head's set: sinks first, then the window.
__device__ __forceinline__ int local_token(const ProbDev& p, int L, int j) {
  const int W = min(p.window, L);
  const int ns = min(p.n_sink, L - W);
  return (j < ns) ? j : (L - W + (j - ns));
}

// A row of `count` entries is cut into nsplit equal splits of at most `target` entries.
__device__ __forceinline__ int nsplit_of(int count, int target) { return (count + target - 1) / target; }
__device__ __forceinline__ int split_size(int count, int target) {
  const int ns = nsplit_of(count, target);
  return ns > 0 ? (count + ns - 1) / ns : 0;
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

// MODE 0: retrieval slots over the LIST; MODE 1: tiles of local heads over sinks + window
template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void attn_decode_kernel(ProbDev p, int rows, const T* __restrict__ q,
                                                               const T* __restrict__ k, const T* __restrict__ v,
                                                               const rtp_selection sel, int* __restrict__ pre,
                                                               float* __restrict__ part) {
  constexpr int mode = MODE;
  constexpr int H = (MODE == 0) ? 1 : kMaxTileHeads;   // heads per row
  extern __shared__ int pre_s[];   // [rows + 1], sized at launch
  __shared__ int idx_s[kSplit];
  __shared__ int wsum_s[kThreads / 64];
  __shared__ int target_s;
  __shared__ float gm_s[kGroups], gl_s[kGroups];
  __shared__ float go_s[kGroups][kHeadDim];
  const int tid = threadIdx.x;
  // split prefix over the rows (every workgroup computes it; block 0 publishes it
  // for the combine kernel): pre[r] = sum of nsplit(count) over rows before r.
  // Rows are dealt to threads round-robin so all their counts load at once.
  {
    constexpr int PR = kMaxRowsLds / kThreads;
    const int nchunks = rows / kThreads + 1;   // chunks holding rows 0..rows
    const int lane = tid & 63, wid = tid >> 6;
    int vv[PR];
    long long tot_entries = 0;
#pragma unroll
    for (int t = 0; t < PR; ++t) {
      const int r = t * kThreads + tid;
      vv[t] = 0;
      if (r < rows) vv[t] = row_info(p, mode, r, sel).count;
      tot_entries += vv[t];
    }
    // target split size: the entries spread over the grid once, within [kMinSplit, kSplit]
    tot_entries = wave_allreduce(tot_entries, OpAdd());
    if (lane == 0) wsum_s[wid] = (int)min(tot_entries, (long long)0x7FFFFFFF);
    __syncthreads();
    if (tid == 0) {
      // sum_r ceil(count_r / t) <= total / t + rows, so t >= total / (grid - rows)
      // puts every split of every row in one round of the grid
      long long te = 0;
      for (int w2 = 0; w2 < kThreads / 64; ++w2) te += wsum_s[w2];
      const long long slots = (long long)gridDim.x - rows;
      long long t = kSplit;
      if (kBalance && slots > 0) t = (te + slots - 1) / slots;
      target_s = (int)min((long long)kSplit, max((long long)kMinSplit, t));
    }
    __syncthreads();
    const int target = target_s;
#pragma unroll
    for (int t = 0; t < PR; ++t) vv[t] = nsplit_of(vv[t], target);
    int carry = 0;
#pragma unroll
    for (int t = 0; t < PR; ++t) {
      if (t >= nchunks) break;
      const int inc = wave_scan_add(vv[t]);   // inclusive, register-only (DPP)
      if (lane == 63) wsum_s[wid] = inc;
      __syncthreads();
      int off = carry, tot = 0;
      for (int w2 = 0; w2 < kThreads / 64; ++w2) {
        if (w2 < wid) off += wsum_s[w2];
        tot += wsum_s[w2];
      }
      const int r = t * kThreads + tid;
      if (r <= rows) pre_s[r] = off + inc - vv[t];
      carry += tot;
      __syncthreads();
    }
    if (blockIdx.x == 0)
      for (int r = tid; r <= rows; r += kThreads) pre[r] = pre_s[r];
  }
  const int total = pre_s[rows];
  const int target = target_s;
  const int grp = tid >> 4, gl = tid & 15;
  const int d0 = gl * 8;
  const size_t kstride = (size_t)p.Hkv * kHeadDim;
  const float qscale = 0.08838834764831845f * kLog2e;   // log2(e) / sqrt(128)

  for (int wi = blockIdx.x; wi < total; wi += gridDim.x) {
    // row of this work item: last r with pre[r] <= wi
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre_s[mid] <= wi) lo = mid; else hi = mid - 1;
    }
    const int row = lo;
    const int split = wi - pre_s[row];
    const RowInfo ri = row_info(p, mode, row, sel);
    const int nh = min(ri.nh, H);
    const int sz = split_size(ri.count, target);
    const int j0 = split * sz;
    const int j1 = min(ri.count, j0 + sz);
    const T* kb = k + ((size_t)ri.k0 * p.Hkv + ri.g) * kHeadDim + d0;
    const T* vb = v + ((size_t)ri.k0 * p.Hkv + ri.g) * kHeadDim + d0;
    // the split's key positions, staged once (coalesced)
    if (mode == 0) {
      const int* list = sel.idx + (size_t)(row / p.batch) * p.Tk + ri.k0;
      for (int j = j0 + tid; j < j1; j += kThreads) idx_s[j - j0] = list[j];
    } else {
      for (int j = j0 + tid; j < j1; j += kThreads) idx_s[j - j0] = key_slot(p, local_token(p, ri.L, j));
    }

    float qv[H][8];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int hh = (h < nh) ? head_of(p, mode, ri, h) : head_of(p, mode, ri, 0);
      RowVec<T> qq;
      qq.load(q + ((size_t)ri.qrow * p.Hq + hh) * kHeadDim + d0);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[h][i] = qq.get(i) * qscale;
    }
    float m[H], l[H], o[H][8];
#pragma unroll
    for (int h = 0; h < H; ++h) {
      m[h] = -INFINITY;
      l[h] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[h][i] = 0.f;
    }
    __syncthreads();

    // two batches of kUnroll tokens per group in flight
    RowVec<T> ka[kUnroll], va[kUnroll], kb2[kUnroll], vb2[kUnroll];
    auto load = [&](RowVec<T>* kr, RowVec<T>* vr, int jb) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = jb + u * kGroups;
        const int n = (j < j1) ? idx_s[j - j0] : idx_s[0];
        kr[u].load(kb + (size_t)n * kstride);
        vr[u].load(vb + (size_t)n * kstride);
      }
    };
    auto compute = [&](const RowVec<T>* kr, const RowVec<T>* vr, int jb) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const bool ok = (jb + u * kGroups) < j1;
#pragma unroll
        for (int h = 0; h < H; ++h) {
          if (h >= nh) break;
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(qv[h][i], kr[u].get(i), a);
          a = row16_sum(a);
          if (ok) {
            const float mn = fmaxf(m[h], a);
            const float sc = __builtin_amdgcn_exp2f(m[h] - mn);
            const float pe = __builtin_amdgcn_exp2f(a - mn);
            l[h] = l[h] * sc + pe;
#pragma unroll
            for (int i = 0; i < 8; ++i) o[h][i] = fmaf(pe, vr[u].get(i), o[h][i] * sc);
            m[h] = mn;
          }
        }
      }
    };
    const int jfirst = j0 + grp;
    if (jfirst < j1) load(ka, va, jfirst);
    for (int jb = jfirst; jb < j1; jb += 2 * kStep) {
      const bool has_b = jb + kStep < j1;
      if (has_b) load(kb2, vb2, jb + kStep);
      compute(ka, va, jb);
      if (jb + 2 * kStep < j1) load(ka, va, jb + 2 * kStep);
      if (has_b) compute(kb2, vb2, jb + kStep);
    }

    // merge the 16 groups of the workgroup, one head at a time
#pragma unroll
    for (int h = 0; h < H; ++h) {
      if (h >= nh) break;
      if (gl == 0) { gm_s[grp] = m[h]; gl_s[grp] = l[h]; }
#pragma unroll
      for (int i = 0; i < 8; ++i) go_s[grp][d0 + i] = o[h][i];
      __syncthreads();
      float* rec = part + ((size_t)wi * H + h) * kPart;
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
}

// Log-sum-exp merge of a (row, head)'s split partials: split weights first (one
// load per thread), then every thread sums its head dim over the splits with
// independent loads.
template <typename T, int MODE>
__global__ __launch_bounds__(kHeadDim) void attn_decode_combine(ProbDev p, const rtp_selection sel,
                                                                const int* __restrict__ pre,
                                                                const float* __restrict__ part,
                                                                T* __restrict__ out, float* __restrict__ lse) {
  constexpr int mode = MODE;
  constexpr int H = (MODE == 0) ? 1 : kMaxTileHeads;
  constexpr int kMaxS = 256;
  __shared__ float wgt_s[kMaxS];
  __shared__ float red_s[2], red2_s[2];
  __shared__ float sum_s;
  const int row = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x;
  const RowInfo ri = row_info(p, mode, row, sel);
  if (h >= ri.nh) return;
  const int head = head_of(p, mode, ri, h);
  const int s0 = pre[row], s1 = pre[row + 1];
  const int ns = s1 - s0;
  auto rec_of = [&](int s) { return part + ((size_t)(s0 + s) * H + h) * kPart; };
  float acc = 0.f, M = -INFINITY, sum = 0.f;
  for (int c0 = 0; c0 < ns; c0 += kMaxS) {
    const int cn = min(kMaxS, ns - c0);
    // the first 32 splits' partial outputs do not depend on the weights: requested
    // with the split maxima, so both arrive in one round trip
    float v32[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v32[u] = (u < cn) ? rec_of(c0 + u)[2 + tid] : 0.f;
    // block max of the split maxima of this chunk
    float mloc = -INFINITY;
    for (int s = tid; s < cn; s += kHeadDim) mloc = fmaxf(mloc, rec_of(c0 + s)[0]);
    mloc = wave_max(mloc);
    if ((tid & 63) == 0) red_s[tid >> 6] = mloc;
    __syncthreads();
    const float mc = fmaxf(red_s[0], red_s[1]);
    const float Mn = fmaxf(M, mc);
    const float scale = __builtin_amdgcn_exp2f(M - Mn);
    acc *= scale;
    sum *= scale;
    M = Mn;
    float sl = 0.f;
    for (int s = tid; s < cn; s += kHeadDim) {
      const float* r = rec_of(c0 + s);
      const float wv = __builtin_amdgcn_exp2f(r[0] - M);
      wgt_s[s] = wv;
      sl = fmaf(r[1], wv, sl);
    }
    sl = wave_sum(sl);
    if ((tid & 63) == 0) red2_s[tid >> 6] = sl;
    __syncthreads();
    if (tid == 0) sum_s = red2_s[0] + red2_s[1];
    // 32 independent loads in flight, summed in split order
    for (int s = 0; s < cn; s += 32) {
      if (s > 0) {
#pragma unroll
        for (int u = 0; u < 32; ++u) v32[u] = (s + u < cn) ? rec_of(c0 + s + u)[2 + tid] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (s + u < cn) acc = fmaf(v32[u], wgt_s[s + u], acc);
    }
    __syncthreads();
    sum += sum_s;
    __syncthreads();
  }
  out[((size_t)ri.qrow * p.Hq + head) * kHeadDim + tid] = Elem<T>::from_f(acc / sum);
  if (lse && tid == 0) lse[(size_t)head * p.Tq + ri.qrow] = (M + __log2f(sum)) * 0.6931471805599453f;
}

// ---- bfloat16, a KV group's heads together on the matrix cores (group_decode):
//   local heads: a row is (tile of up to kGH local heads of one KV group,
//     sequence) over the sinks + window list, in chunks of kGChunk keys;
//   retrieval heads, when a group holds two or more of them: a row is (tile of
//     the group's retrieval heads, sequence) over the union of their LISTs
//     (each K/V row of the group is read once for all heads that selected it,
//     the group-wise loading of "Full Attention Strikes Back ...", paper-graph-ui
//     summary, Table 6), in ranges of kUR positions: the range's entries of each
//     head's LIST (located through a boundary table) mark the positions in LDS,
//     the marked positions form the chunk and a (head, key) pair outside the
//     head's LIST is masked out.
// A row's chunks are dealt round-robin to nsplit one-wave workgroups.  Per chunk
// the wave
//   - issues every load first: K rows straight into MFMA operand layout and
//     the V rows (16 lanes per row), so it waits on memory once;
//   - scores the keys against the tile's heads with 16x16x32 MFMAs (A = K,
//     B = the heads' queries),
//   - updates every head's running max and sum (16-lane groups of the output
//     layout hold one head's scores) and stores the chunk's weights and V rows
//     in LDS,
//   - accumulates P V on the vector ALUs: lane (dims 8c..8c+7, heads 2j, 2j+1)
//     reads each V row segment and the two weights from LDS.
// Splits write (max, sum, o) partials that a second kernel merges by
// log-sum-exp, as for the other decode rows.
constexpr int kGH = 8;           // local heads per tile
constexpr int kGChunk = 32;      // keys per chunk
static_assert(kGChunk % 16 == 0 && kGChunk <= 64, "16-key MFMA tiles; one slot per lane");
constexpr int kGMaxSplit = 64;   // splits per row at most
constexpr int kGTargetWaves = 2048;

constexpr int kUR = 64;          // positions per range of the retrieval union path

// Boundaries of every retrieval slot's LIST in ranges of kUR positions:
// bnd[(r * batch + b) * (nr + 1) + s] = the first list entry at a position >= s * kUR
// (the list is ascending), for s = 0 .. ceil(L / kUR).
__global__ __launch_bounds__(256) void ret_union_bounds(ProbDev p, rtp_selection sel, int nr,
                                                        int* __restrict__ bnd) {
  const int row = blockIdx.y;
  const int r = row / p.batch, b = row % p.batch;
  const int L = p.cu_k[b + 1] - p.cu_k[b];
  const int nrng = (L + kUR - 1) / kUR;
  const int count = min(sel.count[(size_t)r * p.Tq + p.cu_q[b]], L);
  const int* list = sel.idx + (size_t)r * p.Tk + key_row0(p, b);
  int* B = bnd + (size_t)row * (nr + 1);
  auto range_of = [&](int i) { return min(max(list[i], 0) / kUR, max(nrng - 1, 0)); };
  if (count <= 0) {
    for (int t = blockIdx.x * 256 + threadIdx.x; t <= nrng; t += gridDim.x * 256) B[t] = 0;
    return;
  }
  for (int i = blockIdx.x * 256 + threadIdx.x; i < count; i += gridDim.x * 256) {
    const int s = range_of(i);
    const int sp = (i == 0) ? -1 : range_of(i - 1);
    for (int t = sp + 1; t <= s; ++t) B[t] = i;
    if (i == count - 1)
      for (int t = s + 1; t <= nrng; ++t) B[t] = count;
  }
}

// RET = false: a tile of local heads over sinks + window, chunks of kGChunk keys.
// RET = true: a tile of retrieval heads of one KV group over the union of their
// LISTs, chunks = ranges of kUR positions; a (head, key) pair outside the head's
// LIST is masked out.
template <bool RET>
__global__ __launch_bounds__(64) void group_decode(ProbDev p, int nsplit, int nr, const bf16_t* __restrict__ q,
                                                   const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                   const rtp_selection sel, const int* __restrict__ bnd,
                                                   float* __restrict__ part) {
  constexpr int CH = RET ? kUR : kGChunk;   // keys (positions) per chunk
  const int split = blockIdx.x, row = blockIdx.y;
  const int b = row % p.batch, tile = row / p.batch;
  const int lane = threadIdx.x, col = lane & 15, g = lane >> 4;
  const int L = p.cu_k[b + 1] - p.cu_k[b];
  const int W = min(p.window, L);
  const int ns = min(p.n_sink, L - W);
  const int count = RET ? L : ns + W;       // positions walked
  const int nchunk = (count + CH - 1) / CH;
  if (split >= min(nsplit, nchunk)) return;
  const int nh = RET ? p.rtile_cnt[tile] : p.gtile_cnt[tile];
  const int h0 = RET ? p.rtile_start[tile] : p.gtile_start[tile];
  auto head_at = [&](int i) { return RET ? p.ret_heads[h0 + i] : p.local_heads[h0 + i]; };
  const int kvg = kv_of(p, head_at(0));
  const int qrow = p.cu_q[b];
  const size_t kstride = (size_t)p.Hkv * kHeadDim;
  const bf16_t* kb = k + ((size_t)key_row0(p, b) * p.Hkv + kvg) * kHeadDim;
  const bf16_t* vb = v + ((size_t)key_row0(p, b) * p.Hkv + kvg) * kHeadDim;
  const float qscale = 0.08838834764831845f * kLog2e;   // log2(e) / sqrt(128)

  __shared__ int slot_s[CH];
  __shared__ uint32_t hm_s[RET ? CH : 1];    // union: heads selecting position c * CH + i
  __shared__ uint32_t um_s[RET ? CH : 1];    // union: heads selecting the chunk's key j
  __shared__ __attribute__((aligned(16))) float p_s[CH][kGH];
  __shared__ float scale_s[kGH];
  __shared__ __attribute__((aligned(16))) bf16_t v_s[CH][kHeadDim + 8];   // the chunk's V rows

  // B operand: column = head slot col (zero past the tile), k = dims 32 kc + 8 g .. + 8
  FragBF16 qf[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) {
    if (col < nh) {
      load_frag(qf[kc], q + ((size_t)qrow * p.Hq + head_at(col)) * kHeadDim + 32 * kc + 8 * g);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[kc].v[e] = (__bf16)0.f;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;   // head col (output layout)
  const int dc = lane & 15, hg = lane >> 4;
  float o[2][8];                           // heads 2 hg, 2 hg + 1; dims 8 dc .. + 8
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[u][e] = 0.f;

  for (int c = split; c < nchunk; c += nsplit) {
    int nv;
    if (RET) {
      // the range's entries of every head's LIST mark the positions they select
      if (lane < CH) hm_s[lane] = 0u;
      __syncthreads();
      for (int hh = 0; hh < nh; ++hh) {
        const int* Bh = bnd + (size_t)((h0 + hh) * p.batch + b) * (nr + 1);
        const int* list = sel.idx + (size_t)(h0 + hh) * p.Tk + key_row0(p, b);
        const int e1 = Bh[c + 1];
        for (int i = Bh[c] + lane; i < e1; i += 64) {
          const int d = list[i] - c * CH;
          if (d >= 0 && d < CH) atomicOr(&hm_s[d], 1u << hh);
        }
      }
      __syncthreads();
      const uint32_t mk = (lane < CH) ? hm_s[lane] : 0u;
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(mk != 0u);
      nv = __popcll(bal);
      if (mk) {
        const int at = __popcll(bal & ((1ull << lane) - 1ull));
        slot_s[at] = c * CH + lane;
        um_s[at] = mk;
      }
      __syncthreads();
      if (nv == 0) continue;   // no head selects a key of this range
      if (lane < CH && lane >= nv) slot_s[lane] = slot_s[nv - 1];
      __syncthreads();
    } else {
      const int j0 = c * CH;
      nv = min(CH, count - j0);   // valid keys of the chunk (>= 1)
      if (lane < CH) slot_s[lane] = key_slot(p, local_token(p, L, j0 + min(lane, nv - 1)));
      __syncthreads();
    }
    // every load of the chunk first: K in operand layout, V rows (16 lanes per row,
    // key (lane >> 4) + 4 u), so the chunk waits on memory once
    constexpr int NT = CH / 16;   // 16-key tiles of a chunk
    FragBF16 kf[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16_t* kr = kb + (size_t)slot_s[16 * t + col] * kstride + 8 * g;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) load_frag(kf[t][kc], kr + 32 * kc);
    }
    uint4 vr[CH / 4];
#pragma unroll
    for (int u = 0; u < CH / 4; ++u)
      vr[u] = *reinterpret_cast<const uint4*>(vb + (size_t)slot_s[g + 4 * u] * kstride + 8 * col);
    // scores: tile t holds keys 16 t .. 16 t + 15 (rows) x heads (columns)
    f32x4 sc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) sc[t] = mma_k32(kf[t][kc], qf[kc], sc[t]);
    }
    // lane (col, g) holds keys 16 t + 4 g + i of head col
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * t + 4 * g + i;
        bool ok = j < nv;
        if (RET) ok = ok && ((um_s[j] >> col) & 1u);
        sc[t][i] = ok ? sc[t][i] * qscale : -INFINITY;
        mx = fmaxf(mx, sc[t][i]);
      }
    mx = col4_max(mx);
    const float mn = fmaxf(m_run, mx);
    const float mref = (mn == -INFINITY) ? 0.f : mn;   // a head with no key yet keeps l = 0
    const float rs = __builtin_amdgcn_exp2f(m_run - mref);
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pe = __builtin_amdgcn_exp2f(sc[t][i] - mref);
        ls += pe;
        if (col < kGH) p_s[16 * t + 4 * g + i][col] = pe;
      }
    ls = col4_sum(ls);
    l_run = l_run * rs + ls;
    m_run = mn;
    if (g == 0 && col < kGH) scale_s[col] = rs;
#pragma unroll
    for (int u = 0; u < CH / 4; ++u) *reinterpret_cast<uint4*>(&v_s[g + 4 * u][8 * col]) = vr[u];
    __syncthreads();
    // P V: lane (dc, hg) over the chunk's valid keys (weights of masked keys are 0)
    {
      const float r0 = scale_s[2 * hg], r1 = scale_s[2 * hg + 1];
#pragma unroll
      for (int e = 0; e < 8; ++e) { o[0][e] *= r0; o[1][e] *= r1; }
    }
#pragma unroll 4
    for (int j = 0; j < nv; ++j) {
      const uint4 vv = *reinterpret_cast<const uint4*>(&v_s[j][8 * dc]);
      const float2 pw = *reinterpret_cast<const float2*>(&p_s[j][2 * hg]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t wd = (&vv.x)[e >> 1];
        const float ve = __uint_as_float((e & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
        o[0][e] = fmaf(pw.x, ve, o[0][e]);
        o[1][e] = fmaf(pw.y, ve, o[1][e]);
      }
    }
    __syncthreads();
  }
  float* rec0 = part + ((size_t)row * nsplit + split) * kGH * kPart;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int h = 2 * hg + u;
    if (h < nh) {
      float* rec = rec0 + (size_t)h * kPart + 2 + 8 * dc;
#pragma unroll
      for (int e = 0; e < 8; ++e) rec[e] = o[u][e];
    }
  }
  if (g == 0 && col < nh) {
    rec0[(size_t)col * kPart] = m_run;
    rec0[(size_t)col * kPart + 1] = l_run;
  }
}

// Log-sum-exp merge of one (row, head)'s split partials: thread s < S reads split
// s's (max, sum), the block forms the weights, then every thread (one head dim)
// sums its dim over the splits, 32 independent loads at a time.
template <bool RET>
__global__ __launch_bounds__(kHeadDim) void group_decode_combine(ProbDev p, int nsplit,
                                                                 const float* __restrict__ part,
                                                                 bf16_t* __restrict__ out,
                                                                 float* __restrict__ lse) {
  static_assert(kGMaxSplit <= kHeadDim, "one thread per split");
  const int row = blockIdx.x / kGH, h = blockIdx.x % kGH;
  const int b = row % p.batch, tile = row / p.batch;
  if (h >= (RET ? p.rtile_cnt[tile] : p.gtile_cnt[tile])) return;
  const int tid = threadIdx.x;
  const int head = RET ? p.ret_heads[p.rtile_start[tile] + h] : p.local_heads[p.gtile_start[tile] + h];
  const int L = p.cu_k[b + 1] - p.cu_k[b];
  const int W = min(p.window, L);
  const int count = RET ? L : min(p.n_sink, L - W) + W;
  const int CH = RET ? kUR : kGChunk;
  const int S = min(nsplit, (count + CH - 1) / CH);
  const int qrow = p.cu_q[b];
  const float* rec0 = part + (size_t)row * nsplit * kGH * kPart + (size_t)h * kPart;
  const size_t sstride = (size_t)kGH * kPart;
  __shared__ float w_s[kGMaxSplit];
  __shared__ float red_s[kHeadDim / 64];
  __shared__ float red2_s[kHeadDim / 64];
  const float ms = (tid < S) ? rec0[tid * sstride] : -INFINITY;
  const float ls = (tid < S) ? rec0[tid * sstride + 1] : 0.f;
  float mx = wave_max(ms);
  if ((tid & 63) == 0) red_s[tid >> 6] = mx;
  __syncthreads();
  float M = red_s[0];
#pragma unroll
  for (int w2 = 1; w2 < kHeadDim / 64; ++w2) M = fmaxf(M, red_s[w2]);
  const float wv = (tid < S && ms != -INFINITY) ? __builtin_amdgcn_exp2f(ms - M) : 0.f;
  if (tid < kGMaxSplit) w_s[tid] = wv;
  float sl = wave_sum(ls * wv);
  if ((tid & 63) == 0) red2_s[tid >> 6] = sl;
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int w2 = 0; w2 < kHeadDim / 64; ++w2) sum += red2_s[w2];
  float acc = 0.f;
  for (int s0 = 0; s0 < S; s0 += 32) {
    float v32[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v32[u] = (s0 + u < S) ? rec0[(s0 + u) * sstride + 2 + tid] : 0.f;
#pragma unroll
    for (int u = 0; u < 32; ++u)
      if (s0 + u < S) acc = fmaf(v32[u], w_s[s0 + u], acc);
  }
  const bool none = !(sum > 0.f);   // no key at all (an empty set): zeros, lse = -inf
  out[((size_t)qrow * p.Hq + head) * kHeadDim + tid] = Elem<bf16_t>::from_f(none ? 0.f : acc / sum);
  if (lse && tid == 0) lse[(size_t)head * p.Tq + qrow] = none ? -INFINITY : (M + __log2f(sum)) * 0.6931471805599453f;
}

// splits per row of the bfloat16 local path: about kGTargetWaves waves in all
inline int gqa_nsplit(const ProbDev& p) {
  const int rows = p.n_gtiles * p.batch;
  const int cnt = min(p.window, p.max_k) + p.n_sink;
  const int nchunk = max(1, (cnt + kGChunk - 1) / kGChunk);
  const int want = (kGTargetWaves + max(rows, 1) - 1) / max(rows, 1);
  return max(1, min(min(nchunk, kGMaxSplit), want));
}
inline size_t ws_gqa(const ProbDev& p) {
  return sizeof(float) * (size_t)p.n_gtiles * p.batch * gqa_nsplit(p) * kGH * kPart;
}
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// the retrieval union path: groups holding two or more retrieval heads (bfloat16)
inline bool use_union(const ProbDev& p, bool bf16) { return bf16 && p.max_rtile >= 2; }
inline int union_nr(const ProbDev& p) { return max(1, (p.max_k + kUR - 1) / kUR); }
inline int union_nsplit(const ProbDev& p) {
  const int rows = p.n_rtiles * p.batch;
  const int want = (kGTargetWaves + max(rows, 1) - 1) / max(rows, 1);
  return max(1, min(min(union_nr(p), kGMaxSplit), want));
}
inline size_t ws_union_bnd(const ProbDev& p) {
  return align256(sizeof(int) * (size_t)p.R * p.batch * (union_nr(p) + 1));
}
inline size_t ws_union(const ProbDev& p) {
  return ws_union_bnd(p) + sizeof(float) * (size_t)p.n_rtiles * p.batch * union_nsplit(p) * kGH * kPart;
}


inline int rows_of(const ProbDev& p, int mode) { return ((mode == 0) ? p.R : p.n_ltiles) * p.batch; }
inline int heads_per_row(int mode) { return (mode == 0) ? 1 : kMaxTileHeads; }

// Resident workgroups of one launch (the grid), from the device's CU count.
inline int resident_grid() {
  int n_cu = 256, dev = 0, cu = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
    n_cu = cu;
  return n_cu * kWgPerCu;
}

// Upper bound on the number of splits.  While the target is ceil(total / (grid -
// rows)) (or is raised to kMinSplit), sum_r ceil(count_r / target) <= total /
// target + rows <= grid.  When it is capped at kSplit, a row has ceil(count /
// kSplit) splits, bounded through count <= L_b.
inline size_t max_work(const ProbDev& p, int mode, int rows) {
  size_t capped;
  if (mode == 1) {
    const int cnt = min(p.window, p.max_k) + p.n_sink;
    capped = (size_t)rows * ((cnt + kSplit - 1) / kSplit);
  } else {
    const size_t per_row = (size_t)(p.max_k + kSplit - 1) / kSplit;
    const size_t by_total = (size_t)((p.Tk + kSplit - 1) / kSplit) + (size_t)p.batch;  // sum over sequences
    capped = (size_t)(rows / max(1, p.batch)) * min(per_row * p.batch, by_total);
  }
  return max(capped, (size_t)resident_grid());
}

}  // namespace

// ---- scratch of the entry point that allocates nothing (rtp_sparse_attn_decode_noalloc).
// One copy per device, kept until the process ends; every call on a device shares it.
// The decode attention kernels write each workspace word before reading it, so
// nothing needs clearing between calls.
namespace {
constexpr size_t kScratchBytes = RTP_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // the array's device address, per device
}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // with this device current: the symbol's address in this device's copy of the module
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int attn_decode_max_rows() { return kMaxRowsLds - 1; }
int attn_decode_tile_heads() { return kMaxTileHeads; }
int attn_decode_group_heads() { return kGH; }

size_t ws_attn_decode(const ProbDev& p, int mode) {
  const int rows = rows_of(p, mode);
  const size_t split_list = align256(sizeof(int) * (size_t)(rows + 1)) +
                            sizeof(float) * max_work(p, mode, rows) * heads_per_row(mode) * kPart;
  // local heads: float32 takes the split-list kernel, bfloat16 the group kernel; retrieval
  // heads: the split-list kernel, or the union kernel when a group holds two or more (bfloat16)
  if (mode == 1) return max(split_list, ws_gqa(p));
  return p.max_rtile >= 2 ? max(split_list, ws_union(p)) : split_list;
}

hipError_t launch_attn_decode(const ProbDev& p, bool bf16, int mode, const void* q, const void* k,
                              const void* v, const rtp_selection* sel, void* out, float* lse, void* ws,
                              hipStream_t s) {
  const int rows = rows_of(p, mode);
  if (rows == 0) return hipSuccess;
  if (mode == 1 && bf16) {
    const int grows = p.n_gtiles * p.batch;
    const int nsplit = gqa_nsplit(p);
    float* part = (float*)ws;
    const rtp_selection none = {};
    hipLaunchKernelGGL(group_decode<false>, dim3(nsplit, grows), dim3(64), 0, s, p, nsplit, 0, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, none, (const int*)nullptr, part);
    hipLaunchKernelGGL(group_decode_combine<false>, dim3(grows * kGH), dim3(kHeadDim), 0, s, p, nsplit,
                       (const float*)part, (bf16_t*)out, lse);
    return hipGetLastError();
  }
  if (mode == 0 && use_union(p, bf16)) {
    const int rrows = p.n_rtiles * p.batch;
    const int nsplit = union_nsplit(p), nr = union_nr(p);
    int* bnd = (int*)ws;
    float* part = (float*)((char*)ws + ws_union_bnd(p));
    const unsigned bgrid = (unsigned)max(1, (p.max_k + 255) / 256);
    hipLaunchKernelGGL(ret_union_bounds, dim3(bgrid, p.R * p.batch), dim3(256), 0, s, p, *sel, nr, bnd);
    hipLaunchKernelGGL(group_decode<true>, dim3(nsplit, rrows), dim3(64), 0, s, p, nsplit, nr, (const bf16_t*)q,
                       (const bf16_t*)k, (const bf16_t*)v, *sel, (const int*)bnd, part);
    hipLaunchKernelGGL(group_decode_combine<true>, dim3(rrows * kGH), dim3(kHeadDim), 0, s, p, nsplit,
                       (const float*)part, (bf16_t*)out, lse);
    return hipGetLastError();
  }
  rtp_selection sl = {};
  if (sel) sl = *sel;
  int* pre = (int*)ws;
  float* part = (float*)((char*)ws + align256(sizeof(int) * (size_t)(rows + 1)));
  // a resident grid: every workgroup walks its work items, so the row prefix is
  // computed once per workgroup and no launch round waits on the previous one
  const unsigned grid = (unsigned)resident_grid();
  const size_t lds = sizeof(int) * (size_t)(rows + 1);
  const unsigned cgrid = (unsigned)(rows * heads_per_row(mode));
#define RTP_LAUNCH(TT, MM)                                                                                        \
  do {                                                                                                            \
    hipLaunchKernelGGL((attn_decode_kernel<TT, MM>), dim3(grid), dim3(kThreads), lds, s, p, rows, (const TT*)q,     \
                       (const TT*)k, (const TT*)v, sl, pre, part);                                                \
    hipLaunchKernelGGL((attn_decode_combine<TT, MM>), dim3(cgrid), dim3(kHeadDim), 0, s, p, sl, (const int*)pre,  \
                       part, (TT*)out, lse);                                                                      \
  } while (0)
  if (bf16) {
    if (mode == 0) RTP_LAUNCH(bf16_t, 0); else RTP_LAUNCH(bf16_t, 1);
  } else {
    if (mode == 0) RTP_LAUNCH(float, 0); else RTP_LAUNCH(float, 1);
  }
#undef RTP_LAUNCH
  return hipGetLastError();
}

}  // namespace rtp
