// Prefill attention on matrix cores, for both head kinds.
//
//   MODE 0, retrieval heads: key n is attended by query i iff it is causal and
//     in the top-p set of the row, S = {s_n > tau_i} U {s_n == tau_i, n <= tie_i}
//     ("Full Attention Strikes Back ...", paper-graph-ui summary, section 3.4,
//     Eq. 5 and the attention equation after it).  s_n is recomputed here
//     with the same MFMA indexer tile the selection used, so membership is
//     bit-identical to the selection.
//   MODE 1, local heads: keys n <= pos with pos - n < W, plus sinks n < n_sink
//     (section 3.4 "Local Head Attention Pattern").
//
// The pages give few details of their prefill kernel (retrieval heads run
// dense there); this one is a flash-attention style loop written for gfx950:
//   - workgroup = 8 wave64s, 256 query rows (32 per wave as two 16-column
//     MFMA tiles), 64-key tiles: every staged K/V tile feeds 256 queries, which
//     halves the re-reads of the causal K/V prefix against 128-row tiles
//     (a 4-wave, 128-row variant needs more than 128 VGPRs per lane and
//     spills at two workgroups per CU);
//   - a later tile's K/V is loaded into registers while the current one is
//     computed, then written to a free LDS slot: bfloat16 keeps four slots,
//     stages two tiles ahead and synchronises the workgroup every second tile
//     (between barriers a wave that finished its tile goes on with the next,
//     beside the slower wave of its SIMD); float32 and the tile-skipping
//     instance keep two slots and a barrier per tile;
//   - S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (f32 path: 16x16x4 steps), K
//     tile staged row-major in LDS; the S^T output layout (a lane holds 4 keys
//     of one query column) is already the B-operand layout of O^T = V^T P^T,
//     so P goes from registers into the second product without a shuffle;
//     V is staged transposed in LDS (rows = head dims) for the A operand;
//   - online softmax in the log2 domain with a reference that moves only when
//     a row maximum exceeds it by more than 8; row sums from the matrix cores
//     (an all-ones operand in the PV product); masked tiles of a wave skip
//     both products.
//   - the two products run at wave priority 0 and the mask/softmax ALU work
//     at 2, so when two waves of a SIMD are ready the one in its ALU phase
//     issues first and the other's matrix-core work overlaps it.
// LDS strides are padded (chosen by measurement) so that fragment reads of one
// phase mostly hit distinct banks; the 16-bit index-key rows are padded to 10
// words, which removed most of the bank conflicts of their 8-byte reads.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace rtp {

namespace {

constexpr int NC = 2;                     // 16-row MFMA column tiles per wave
constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int RW = 16 * NC;               // query rows per wave
constexpr int BQ = RW * kWaves;           // query rows per workgroup
constexpr int KT = 64;          // keys per tile
static_assert((KT / 2) * (kHeadDim / 8) % kThreads == 0, "V staging splits evenly over the workgroup");
static_assert(KT * kHeadDim / 8 % kThreads == 0, "K staging splits evenly over the workgroup");

template <typename T> struct Lds;
template <> struct Lds<bf16_t> { static constexpr int kStr = 128 + 16; static constexpr int vStr = 64 + 4; };
template <> struct Lds<float> { static constexpr int kStr = 128 + 4; static constexpr int vStr = 64 + 4; };

// ---- B operand of O^T += V^T P^T from the four P values of two key subtiles
__device__ __forceinline__ void make_pfrag(FragBF16& f, const float* a, const float* b) {
  uint4 u;
  u.x = pack_bf16x2(a[0], a[1]);
  u.y = pack_bf16x2(a[2], a[3]);
  u.z = pack_bf16x2(b[0], b[1]);
  u.w = pack_bf16x2(b[2], b[3]);
  f.v = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void make_pfrag(FragF32& f, const float* a, const float* b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f.v[i] = a[i]; f.v[4 + i] = b[i]; }
}

// ---- an operand fragment of ones
template <typename F> __device__ __forceinline__ F ones_frag();
template <> __device__ __forceinline__ FragBF16 ones_frag<FragBF16>() {
  FragBF16 f;
  const uint4 u = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bfloat16 1.0 pairs
  f.v = __builtin_bit_cast(bf16x8, u);
  return f;
}
template <> __device__ __forceinline__ FragF32 ones_frag<FragF32>() {
  FragF32 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = 1.f;
  return f;
}

// ---- A operand of O^T += V^T P^T: row d of V^T, keys (4g..4g+3) and (16+4g..16+4g+3)
__device__ __forceinline__ void load_vfrag(FragBF16& f, const bf16_t* rowp) {
  uint2 a = *reinterpret_cast<const uint2*>(rowp);
  uint2 b = *reinterpret_cast<const uint2*>(rowp + 16);
  uint4 u = {a.x, a.y, b.x, b.y};
  f.v = __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ void load_vfrag(FragF32& f, const float* rowp) {
  float4 a = *reinterpret_cast<const float4*>(rowp);
  float4 b = *reinterpret_cast<const float4*>(rowp + 16);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// ---- staging of one 64-key tile: global -> registers (issued early, one tile
// ahead) -> LDS (K row-major, V transposed)
template <typename T> struct Stage;
// bf16: K as 16-byte row chunks (16 lanes per key row); V as pairs of keys x 8
// dims, written transposed as packed key pairs.
template <> struct Stage<bf16_t> {
  static constexpr int kU = KT * kHeadDim / 8 / kThreads;   // 16-byte K chunks per thread
  static constexpr int kVU = (KT / 2) * (kHeadDim / 8) / kThreads;   // (key pair, 8-dim chunk) units per thread
  uint4 k[kU], v[kVU][2];
  __device__ __forceinline__ void load(const bf16_t* kg, const bf16_t* vg, size_t rstride, int nvalid, int tid) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = u * kThreads + tid;
      const int key = e >> 4, ch = e & 15;
      k[u] = {0u, 0u, 0u, 0u};
      if (key < nvalid) k[u] = *reinterpret_cast<const uint4*>(kg + (size_t)key * rstride + ch * 8);
    }
#pragma unroll
    for (int w = 0; w < kVU; ++w) {
      const int e = w * kThreads + tid;
      const int kp = e & 31, dc = e >> 5;   // keys 2kp, 2kp+1; dims 8dc..8dc+7
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = 2 * kp + u;
        v[w][u] = {0u, 0u, 0u, 0u};
        if (key < nvalid) v[w][u] = *reinterpret_cast<const uint4*>(vg + (size_t)key * rstride + dc * 8);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* k_s, bf16_t* vt_s, int tid) const {
    constexpr int KS = Lds<bf16_t>::kStr, VS = Lds<bf16_t>::vStr;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = u * kThreads + tid;
      const int key = e >> 4, ch = e & 15;
      *reinterpret_cast<uint4*>(k_s + key * KS + ch * 8) = k[u];
    }
#pragma unroll
    for (int w = 0; w < kVU; ++w) {
      const int e2 = w * kThreads + tid;
      const int kp = e2 & 31, dc = e2 >> 5;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w0 = (&v[w][0].x)[e >> 1], w1 = (&v[w][1].x)[e >> 1];
        const uint32_t pr = (e & 1) ? ((w0 >> 16) | (w1 & 0xFFFF0000u)) : ((w0 & 0xFFFFu) | (w1 << 16));
        *reinterpret_cast<uint32_t*>(vt_s + (8 * dc + e) * VS + 2 * kp) = pr;
      }
    }
  }
};
template <> struct Stage<float> {
  static constexpr int kU = KT * kHeadDim / 4 / kThreads;   // 16-byte K chunks per thread
  static constexpr int kVU = (KT / 2) * (kHeadDim / 8) / kThreads;
  float4 k[kU];
  float v[kVU][2][8];
  __device__ __forceinline__ void load(const float* kg, const float* vg, size_t rstride, int nvalid, int tid) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = u * kThreads + tid;
      const int key = e >> 5, ch = e & 31;
      k[u] = {0.f, 0.f, 0.f, 0.f};
      if (key < nvalid) k[u] = *reinterpret_cast<const float4*>(kg + (size_t)key * rstride + ch * 4);
    }
#pragma unroll
    for (int w = 0; w < kVU; ++w) {
      const int e = w * kThreads + tid;
      const int kp = e & 31, dc = e >> 5;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int key = 2 * kp + u;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[w][u][i] = 0.f;
        if (key < nvalid) {
          float4 a = *reinterpret_cast<const float4*>(vg + (size_t)key * rstride + dc * 8);
          float4 b = *reinterpret_cast<const float4*>(vg + (size_t)key * rstride + dc * 8 + 4);
          v[w][u][0] = a.x; v[w][u][1] = a.y; v[w][u][2] = a.z; v[w][u][3] = a.w;
          v[w][u][4] = b.x; v[w][u][5] = b.y; v[w][u][6] = b.z; v[w][u][7] = b.w;
        }
      }
    }
  }
  __device__ __forceinline__ void store(float* k_s, float* vt_s, int tid) const {
    constexpr int KS = Lds<float>::kStr, VS = Lds<float>::vStr;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int e = u * kThreads + tid;
      const int key = e >> 5, ch = e & 31;
      *reinterpret_cast<float4*>(k_s + key * KS + ch * 4) = k[u];
    }
#pragma unroll
    for (int w = 0; w < kVU; ++w) {
      const int e2 = w * kThreads + tid;
      const int kp = e2 & 31, dc = e2 >> 5;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float2 o = {v[w][0][e], v[w][1][e]};
        *reinterpret_cast<float2*>(vt_s + (8 * dc + e) * VS + 2 * kp) = o;
      }
    }
  }
};

template <typename T>
__device__ __forceinline__ void store_out4(T* dst, const float* v);
template <>
__device__ __forceinline__ void store_out4<bf16_t>(bf16_t* dst, const float* v) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = u;
}
template <>
__device__ __forceinline__ void store_out4<float>(float* dst, const float* v) {
  *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
}

// Work order: blockIdx -> (query tile, head).  Workgroups are dealt round-robin
// over the 8 XCDs (block id mod 8), and each XCD has its own L2, so the order
// decides which workgroups share K/V tiles in L2:
//   - heads that share KV (local heads of one group) run side by side: the
//     consecutive workgroups of an XCD take all heads of one query tile;
//   - heads on different KV groups (the retrieval heads, one per group) are
//     given XCDs of their own when they divide the 8 XCDs evenly, so all the
//     workgroups resident on an XCD sweep the same head's K/V prefix at about
//     the same time.
// Query tiles go longest-first so the causal tail does not straggle.
struct Work { int b, qt, hidx; bool ok; };
__device__ __forceinline__ Work work_of(int bid, int nheads, int batch, int tiles_per_b, bool per_head_xcd) {
  Work wk;
  const int units = batch * tiles_per_b;
  const int k = bid >> 3, x = bid & 7;
  int unit;
  if (per_head_xcd) {
    const int xpg = 8 / nheads;            // XCDs per head
    wk.hidx = x % nheads;
    unit = k * xpg + x / nheads;
  } else {
    unit = (k / nheads) * 8 + x;
    wk.hidx = k % nheads;
  }
  wk.ok = unit < units;
  wk.b = unit % batch;
  wk.qt = tiles_per_b - 1 - unit / batch;
  return wk;
}
__host__ __device__ inline bool per_head_xcd(int mode, int nheads) { return mode == 0 && nheads <= 8 && 8 % nheads == 0; }

// MODE 0: retrieval heads, masked-dense tiles; MODE 2: retrieval heads whose rows
// keep under a quarter of their prefix, membership tested before the products so
// that tiles without a selected pair are skipped; MODE 1: local heads.  Modes 0
// and 2 run on the same grid and every workgroup is taken by exactly one of them.
template <typename T, int MODE>
__global__ __launch_bounds__(kThreads, 1) void attn_prefill_kernel(
    ProbDev p, int nheads, int tiles_per_b, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const T* __restrict__ k_idx, const rtp_selection sel, T* __restrict__ out,
    float* __restrict__ lse) {
  typedef typename Frag32<T>::type F;
  typedef typename IdxFrag<T>::type IF;
  constexpr bool kRet = MODE != 1;   // retrieval heads
  constexpr int KS = Lds<T>::kStr, VS = Lds<T>::vStr;
  // LDS tile slots: bfloat16 outside MODE 2 keeps four and synchronises the
  // workgroup every second tile (tiles are staged two ahead); otherwise two, every tile
  constexpr int NBUF = (sizeof(T) == 2 && MODE != 2) ? 4 : 2;
  constexpr int kSync = NBUF / 2;   // tiles per barrier = staging distance
  __shared__ __attribute__((aligned(16))) T k_s[NBUF][KT * KS];
  __shared__ __attribute__((aligned(16))) T vt_s[NBUF][kHeadDim * VS];
  // retrieval heads: the tile's 16-dim index keys, staged with its K/V into the same slot
  constexpr int KXW = kRet ? KT * kIdxDim * (int)sizeof(T) / 4 / kThreads : 0;   // words per thread
  // rows of 16-bit index keys padded to 10 words, so the 16 rows a fragment read
  // touches fall in distinct banks
  constexpr int KXWK = kIdxDim * (int)sizeof(T) / 4;                     // words per key
  constexpr int KXS = (sizeof(T) == 2) ? KXWK + 2 : KXWK;                 // row stride in words
  __shared__ __attribute__((aligned(16))) uint32_t kx_s[NBUF][kRet ? KT * KXS : 1];
  uint32_t kxr[KXW > 0 ? KXW : 1] = {};

  const Work wk = work_of(blockIdx.x, nheads, p.batch, tiles_per_b, per_head_xcd(kRet ? 0 : 1, nheads));
  if (!wk.ok) return;
  const int b = wk.b, hidx = wk.hidx;
  const int h = kRet ? p.ret_heads[hidx] : p.local_heads[hidx];
  const int g = kv_of(p, h);
  const int q0 = p.cu_q[b], Lq = p.cu_q[b + 1] - q0;
  const int k0 = key_row0(p, b), Lk = p.cu_k[b + 1] - p.cu_k[b];
  const int i0 = wk.qt * BQ;
  if (i0 >= Lq) return;
  const int off = Lk - Lq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const size_t rstride = (size_t)p.Hkv * kHeadDim;
  const T* kg = k + ((size_t)k0 * p.Hkv + g) * kHeadDim;
  const T* vg = v + ((size_t)k0 * p.Hkv + g) * kHeadDim;

  // ---- this wave's query rows: i0 + 32w + 16c + col
  F qf[NC][4];
  int qi[NC], qpos[NC];
  bool qok[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qi[c] = i0 + RW * w + 16 * c + col;
    qok[c] = qi[c] < Lq;
    qpos[c] = off + (qok[c] ? qi[c] : (Lq - 1));
  }
  const int wpos_lo = off + min(i0 + RW * w, Lq - 1);
  const int wpos_hi = off + min(i0 + RW * w + RW - 1, Lq - 1);
  IF qxf[NC];
  float tau4[NC];
  int tie[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) { tau4[c] = 0.f; tie[c] = 0; }
  bool exact_ties = false;
  bool all_keys = false;
  const T* kxb = nullptr;
  const int wt_last = wpos_hi / KT;
  // does any row of this wave select a pair in key tile t? (wave-uniform)  Below the
  // wave's lowest row and without exact ties a tile is needed iff its largest dot product
  // reaches some row's threshold; on the diagonal or with ties each pair is tested.
  auto load_tile = [&](IF (&dst)[4], int t) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int key = min(t * KT + 16 * ks + col, Lk - 1);
      load_idx_frag(dst[ks], kxb + (size_t)key * kIdxDim + 4 * grp);
    }
  };
  auto tile_hit = [&](const IF (&src)[4], int t) -> bool {
    if (t > wt_last) return false;
    bool hit = false;
    if (!exact_ties && t * KT + KT - 1 <= wpos_lo) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float mx = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const f32x4 dx = idx_dot_tile(src[ks], qxf[c]);
          mx = fmaxf(mx, fmaxf(fmaxf(dx[0], dx[1]), fmaxf(dx[2], dx[3])));
        }
        hit |= mx >= tau4[c];
      }
    } else {
      const int kb4 = t * KT + 4 * grp;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const f32x4 dx = idx_dot_tile(src[ks], qxf[c]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb4 + 16 * ks + i;
            const bool ok = (dx[i] > tau4[c]) | ((dx[i] == tau4[c]) & (key <= tie[c]));
            hit |= ok & (key <= qpos[c]);
          }
        }
    }
    return __builtin_amdgcn_ballot_w64(hit) != 0ull;
  };
  if (kRet) {
    bool dense_row = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const size_t qr = (size_t)hidx * p.Tq + q0 + (qok[c] ? qi[c] : Lq - 1);
      load_idx_frag(qxf[c], (const T*)sel.q_idx + qr * kIdxDim + 4 * grp);
      tau4[c] = sel.tau[qr] * 4.f;   // compare raw dot products: dot / 4 vs tau is exact
      tie[c] = sel.tie_pos[qr];
      exact_ties |= (tie[c] != 0x7FFFFFFF);
      dense_row |= 4ll * sel.count[qr] >= (long long)qpos[c] + 1;   // keeps a quarter of its prefix or more
    }
    // the workgroup goes to MODE 2 when every row keeps under a quarter of its prefix and
    // the sampled tile union below is sparse (bfloat16 only; float32 is masked-dense)
    __shared__ int wg_dense_s;
    if (tid == 0) wg_dense_s = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(dense_row) != 0 && lane == 0) atomicOr(&wg_dense_s, 1);
    __syncthreads();
    // (and the workgroup's causal range fits the tile list: keys up to 1M)
    const int wg_tiles = (off + min(i0 + BQ, Lq) - 1) / KT + 1;
    const bool wg_sparse = (sizeof(T) == 2) && wg_dense_s == 0 && wg_tiles <= (1 << 14);
    if (MODE == 2 && !wg_sparse) return;
    exact_ties = __builtin_amdgcn_ballot_w64(exact_ties) != 0;
    kxb = k_idx + ((size_t)hidx * p.Tk + k0) * kIdxDim;
    if (wg_sparse) {
      // the tiles' union may still be dense (selections spread over the prefix): 16 tiles
      // spread over the causal range, their index keys loaded at once, decide; more than
      // half of them needed keeps the workgroup on the masked-dense path
      __shared__ uint32_t samp_s;
      if (tid == 0) samp_s = 0u;
      __syncthreads();
      constexpr int kSamp = 16;
      const int ns = min(kSamp, wg_tiles);
      IF kf[kSamp][4];
#pragma unroll
      for (int j = 0; j < kSamp; ++j) load_tile(kf[j], (min(j, ns - 1) * wg_tiles) / ns);
#pragma unroll
      for (int j = 0; j < kSamp; ++j)
        if (j < ns && tile_hit(kf[j], (j * wg_tiles) / ns) && lane == 0) atomicOr(&samp_s, 1u << j);
      __syncthreads();
      const bool union_dense = 2 * __popc(samp_s) > ns;
      if (MODE == 0 && !union_dense) return;
      if (MODE == 2 && union_dense) return;
    }
    // every row of this wave keeps its whole causal prefix (p >= 1, tau = -inf):
    // dense causal attention, no indexer work
    bool rows_all = true;
#pragma unroll
    for (int c = 0; c < NC; ++c) rows_all &= (tau4[c] == -INFINITY);
    all_keys = __builtin_amdgcn_ballot_w64(!rows_all) == 0;
  }
  // (query fragments are loaded once the workgroup is known to run here)
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const T* qp = q + ((size_t)(q0 + (qok[c] ? qi[c] : Lq - 1)) * p.Hq + h) * kHeadDim + 8 * grp;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) load_frag(qf[c][kc], qp + 32 * kc);
  }

  const float sl2 = 0.08838834764831845f * kLog2e;  // log2(e) / sqrt(128)
  float m_[NC];
  // row sums of P on the matrix cores: a constant all-ones A operand turns
  // O^T += V^T P^T into sum_k P[k][row] in every output row (and sums exactly
  // the rounded P that multiplies V)
  f32x4 lacc[NC];
  const F onesf = ones_frag<F>();
  f32x4 oacc[NC][8];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    m_[c] = -INFINITY;
    lacc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- key tiles of the workgroup
  const int pos_lo = off + i0;
  const int pos_hi = off + min(i0 + BQ, Lq) - 1;
  const int kt_last = pos_hi / KT;
  int kt_first = 0;
  bool sink_tile = false;
  if (MODE == 1) {
    kt_first = max(0, pos_lo - p.window + 1) / KT;
    sink_tile = (p.n_sink > 0) && (kt_first > 0);
  }
  int ntiles = kt_last - kt_first + 1 + (sink_tile ? 1 : 0);
  // MODE 2: the key tiles that hold a selected pair for some row of the workgroup,
  // found from the index keys alone (32 bytes a key) before any K/V is staged
  constexpr int kMaxTiles2 = (MODE == 2) ? (1 << 14) : 1;   // keys up to 1M
  __shared__ uint32_t need_s[(kMaxTiles2 + 31) / 32];
  __shared__ unsigned short list_s[kMaxTiles2];
  __shared__ uint32_t nscan_s[kThreads / 64];
  if (MODE == 2) {
    const int nwords = (ntiles + 31) / 32;
    for (int e = tid; e < nwords; e += kThreads) need_s[e] = 0u;
    __syncthreads();
    // every wave tests its rows against each of its causal tiles, three groups of four
    // tiles' index keys in flight
    IF kf[3][4][4];
    auto load4 = [&](IF (&dst)[4][4], int t0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) load_tile(dst[u], t0 + u);
    };
    auto test4 = [&](const IF (&src)[4][4], int t0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (tile_hit(src[u], t0 + u) && lane == 0) atomicOr(&need_s[(t0 + u) >> 5], 1u << ((t0 + u) & 31));
    };
    load4(kf[0], 0);
    load4(kf[1], 4);
    for (int t0 = 0; t0 <= wt_last; t0 += 12) {
      load4(kf[2], t0 + 8);
      test4(kf[0], t0);
      if (t0 + 4 > wt_last) break;
      load4(kf[0], t0 + 12);
      test4(kf[1], t0 + 4);
      if (t0 + 8 > wt_last) break;
      load4(kf[1], t0 + 16);
      test4(kf[2], t0 + 8);
    }
    __syncthreads();
    // the list of needed tiles, ascending: word counts scanned over the workgroup
    uint32_t word = 0u, cnt = 0u;
    if (tid < nwords) { word = need_s[tid]; cnt = (uint32_t)__popc(word); }
    uint32_t inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = __shfl_up(inc, d);
      if (lane >= d) inc += y;
    }
    if (lane == 63) nscan_s[w] = inc;
    __syncthreads();
    uint32_t base = 0u, total = 0u;
    for (int w2 = 0; w2 < kThreads / 64; ++w2) {
      if (w2 < w) base += nscan_s[w2];
      total += nscan_s[w2];
    }
    uint32_t o = base + inc - cnt;
    while (word) {
      const int b = __ffs(word) - 1;
      list_s[o++] = (unsigned short)(32 * tid + b);
      word &= word - 1u;
    }
    ntiles = (int)total;
    __syncthreads();
  }
  auto tile_of = [&](int t) {
    if (MODE == 2) return (int)list_s[t];
    return (sink_tile && t == 0) ? 0 : (kt_first + t - (sink_tile ? 1 : 0));
  };

  // index keys of a tile as 4-byte words (keys past the sequence read as 0)
  auto kx_load = [&](int kb0) {
    if (!kRet) return;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(kxb + (size_t)kb0 * kIdxDim);
    constexpr int kWordsPerKey = kIdxDim * (int)sizeof(T) / 4;
#pragma unroll
    for (int w = 0; w < KXW; ++w) {
      const int e = w * kThreads + tid;
      kxr[w] = (kb0 + e / kWordsPerKey < Lk) ? src[e] : 0u;
    }
  };
  auto kx_store = [&](int b2) {
    if (!kRet) return;
#pragma unroll
    for (int w = 0; w < KXW; ++w) {
      const int e = w * kThreads + tid;
      kx_s[b2][(e / KXWK) * KXS + e % KXWK] = kxr[w];
    }
  };

  Stage<T> st{};   // (zeroed: a slot past the last tile is stored but never read)
#pragma unroll
  for (int j = 0; j < kSync; ++j) {
    if (j < ntiles) {   // (MODE 2 could in principle find no tile: then the rows keep l = 0)
      const int fb = tile_of(j) * KT;
      st.load(kg + (size_t)fb * rstride, vg + (size_t)fb * rstride, rstride, min(KT, Lk - fb), tid);
      kx_load(fb);
    }
    st.store(k_s[j], vt_s[j], tid);
    kx_store(j);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const bool sink_only = sink_tile && (t == 0);
    const int kbase = tile_of(t) * KT;
    const int buf = t % NBUF;
    if (t + kSync < ntiles) {
      const int nb = tile_of(t + kSync) * KT;
      st.load(kg + (size_t)nb * rstride, vg + (size_t)nb * rstride, rstride, min(KT, Lk - nb), tid);
      kx_load(nb);
    }

    // wave-uniform tile classification
    bool skip = kbase > wpos_hi;                                    // all keys in this wave's future
    bool need_mask = kbase + KT - 1 > wpos_lo;                      // crosses the diagonal
    if (MODE == 1) {
      if (sink_only) {
        need_mask = true;
      } else {
        skip |= (kbase + KT - 1) < (wpos_lo - p.window + 1) && kbase >= p.n_sink;  // wholly before every window
        need_mask |= (wpos_hi - kbase) >= p.window;                                // window edge inside
      }
    }
    IF kxf[4];
    if (!skip && kRet && !all_keys) {
      const T* kxt = reinterpret_cast<const T*>(kx_s[buf]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) load_idx_frag(kxf[ks], kxt + (16 * ks + col) * (KXS * 4 / (int)sizeof(T)) + 4 * grp);
    }
    if (!skip) {
      __builtin_amdgcn_s_setprio(0);   // matrix-core phase: waves in their ALU phase issue first
      // S^T = K Q^T
      f32x4 sacc[NC][4];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[c][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* kt_s = k_s[buf];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          F kf;
          load_frag(kf, kt_s + (16 * ks + col) * KS + 32 * kc + 8 * grp);
#pragma unroll
          for (int c = 0; c < NC; ++c) sacc[c][ks] = mma_k32(kf, qf[c][kc], sacc[c][ks]);
        }
      }
      __builtin_amdgcn_s_setprio(2);
      // membership: branch-free masks; the variant (exact ties, boundary tile)
      // is fixed per tile so each inner loop is straight-line code.  Element
      // (ks, i) of a lane is key kb4 + 16 ks + i: the tests compare that
      // compile-time offset with per-row differences computed once per tile
      // (per-element key counters would cost a register and an add each).
      const int kb4 = kbase + 4 * grp;
      int relq[NC], relt[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        relq[c] = opaque_int(qpos[c] - kb4);   // key <= qpos  <=>  16 ks + i <= relq
        relt[c] = opaque_int(tie[c] - kb4);    // key <= tie   <=>  16 ks + i <= relt
      }
      if (kRet) {
        auto apply = [&](auto exact_t, auto mask_t) {
          constexpr bool kExact = decltype(exact_t)::value;
          constexpr bool kMask = decltype(mask_t)::value;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              const f32x4 dx = idx_dot_tile(kxf[ks], qxf[c]);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int ko = 16 * ks + i;
                bool ok;
                if (kExact) ok = (dx[i] > tau4[c]) | ((dx[i] == tau4[c]) & (ko <= relt[c]));
                else ok = dx[i] >= tau4[c];
                if (kMask) ok = ok & (ko <= relq[c]);
                sacc[c][ks][i] = ok ? sacc[c][ks][i] : -INFINITY;
              }
            }
          }
        };
        if (all_keys) {
          if (need_mask) {   // causal mask only
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
              for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  sacc[c][ks][i] = (16 * ks + i <= relq[c]) ? sacc[c][ks][i] : -INFINITY;
          }
        } else if (exact_ties) {
          if (need_mask) apply(std::true_type{}, std::true_type{}); else apply(std::true_type{}, std::false_type{});
        } else {
          if (need_mask) apply(std::false_type{}, std::true_type{}); else apply(std::false_type{}, std::false_type{});
        }
      } else if (need_mask) {
        const int sink_rel = opaque_int(p.n_sink - kb4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ko = 16 * ks + i;
              const bool is_sink = ko < sink_rel;                 // key < n_sink
              const bool in_win = ko > relq[c] - p.window;         // qpos - key < window
              const bool ok = (ko <= relq[c]) & (sink_only ? is_sink : (in_win | is_sink));
              sacc[c][ks][i] = ok ? sacc[c][ks][i] : -INFINITY;
            }
      }

      // online softmax (log2 domain)
      F pf[NC][2];
      bool live = false;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float tmax = -INFINITY;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sacc[c][ks][i]);
        tmax = col4_max(tmax);
        const float mnew = fmaxf(m_[c], tmax * sl2);
        live |= (mnew != -INFINITY);
        // The reference m_ moves (and O, l are rescaled) only when the row maximum
        // exceeds it by more than 8: until then exp2(s - m_) <= 2^8, and O and l
        // keep sharing one reference, so the result is the same.
        const bool up = mnew > m_[c] + 8.f;   // also the first finite maximum
        if (__builtin_amdgcn_ballot_w64(up)) {
          const float mref = up ? mnew : m_[c];
          const float alpha = up ? __builtin_amdgcn_exp2f(m_[c] - mref) : 1.f;
          lacc[c] *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) oacc[c][dt] *= alpha;
          m_[c] = mref;
        }
        const float muse = (m_[c] == -INFINITY) ? 0.f : m_[c];
        float x[4][4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[ks][i] = __builtin_amdgcn_exp2f(fmaf(sacc[c][ks][i], sl2, -muse));
        make_pfrag(pf[c][0], x[0], x[1]);
        make_pfrag(pf[c][1], x[2], x[3]);
      }

      // O^T += V^T P^T; the eight V^T fragments of a 32-key step are read before
      // its products, so the LDS reads overlap instead of each waiting alone
      __builtin_amdgcn_s_setprio(0);
      if (__builtin_amdgcn_ballot_w64(live)) {
        const T* vtt = vt_s[buf];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          F vf[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) load_vfrag(vf[dt], vtt + (16 * dt + col) * VS + 32 * kk + 4 * grp);
          __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the products
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int c = 0; c < NC; ++c) oacc[c][dt] = mma_k32(vf[dt], pf[c][kk], oacc[c][dt]);
#pragma unroll
          for (int c = 0; c < NC; ++c) lacc[c] = mma_k32(onesf, pf[c][kk], lacc[c]);
        }
      }
    }
    __builtin_amdgcn_s_setprio(2);
    // the tile kSync ahead goes to the slot of tile t + kSync - NBUF, which every wave
    // finished before the last barrier; it is visible after the next one
    if (t + kSync < ntiles) {
      const int nbuf = (t + kSync) % NBUF;
      st.store(k_s[nbuf], vt_s[nbuf], tid);
      kx_store(nbuf);
    }
    if ((t + 1) % kSync == 0) __syncthreads();
  }

  // ---- normalise and store
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float lt = lacc[c][0];   // every output row of the ones tile holds the row sum
    if (!qok[c]) continue;
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
    T* op = out + ((size_t)(q0 + qi[c]) * p.Hq + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = oacc[c][dt][i] * inv;
      store_out4<T>(op + 16 * dt + 4 * grp, vv);
    }
    if (lse && grp == 0) lse[(size_t)h * p.Tq + q0 + qi[c]] = (m_[c] + __log2f(lt)) * 0.6931471805599453f;
  }
}

}  // namespace

hipError_t launch_attn_prefill(const ProbDev& p, bool bf16, int mode, const void* q, const void* k,
                               const void* v, const void* k_idx, const rtp_selection* sel, void* out,
                               float* lse, hipStream_t s) {
  const int nheads = (mode == 0) ? p.R : p.n_local;
  if (nheads == 0 || p.Tq == 0) return hipSuccess;
  const int tiles_per_b = (p.max_q + BQ - 1) / BQ;
  const int units = tiles_per_b * p.batch;
  const unsigned nblk = per_head_xcd(mode, nheads) ? 8u * (unsigned)((units + 8 / nheads - 1) / (8 / nheads))
                                                  : (unsigned)(((units + 7) / 8) * 8 * nheads);
  dim3 grid(nblk);
  rtp_selection sl = {};
  if (sel) sl = *sel;
#define RTP_LAUNCH(TT, MM)                                                                                    \
  hipLaunchKernelGGL((attn_prefill_kernel<TT, MM>), grid, dim3(kThreads), 0, s, p, nheads, tiles_per_b,       \
                     (const TT*)q, (const TT*)k, (const TT*)v, (const TT*)k_idx, sl, (TT*)out, lse)
  if (bf16) {
    if (mode == 0) {
      RTP_LAUNCH(bf16_t, 0);
      RTP_LAUNCH(bf16_t, 2);   // the workgroups whose rows are sparse
    } else {
      RTP_LAUNCH(bf16_t, 1);
    }
  } else {
    if (mode == 0) RTP_LAUNCH(float, 0); else RTP_LAUNCH(float, 1);
  }
#undef RTP_LAUNCH
  return hipGetLastError();
}

}  // namespace rtp
