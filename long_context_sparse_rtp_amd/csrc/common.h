// Shared device helpers for the gfx950 kernels: element types, conversions,
// MFMA tile wrappers and wave-level reductions.  Nothing here is specific to
// one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtp {

typedef uint16_t bf16_t;  // bfloat16 bit pattern
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kIdxDim = 16;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ conversions
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round-to-nearest-even float -> bfloat16 (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Two floats -> two packed bfloat16 (hardware round-to-nearest-even on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// Correctly rounded float64 -> bfloat16: keep 8 significant bits with
// round-half-even applied directly to the double's 52-bit fraction (one
// rounding); the bfloat16 subnormal range uses the fixed quantum 2^-133.
__device__ __forceinline__ bf16_t f64_to_bf16_rne(double x) {
  double ax = fabs(x);
  if (ax < 1.1754943508222875e-38) {  // below 2^-126: fixed quantum 2^-133
    double q = ldexp(rint(ldexp(x, 133)), -133);
    return (bf16_t)(__float_as_uint((float)q) >> 16);
  }
  uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint64_t drop = (1ull << 45) - 1ull;  // 52 - 7 fraction bits dropped
  u += (drop >> 1) + ((u >> 45) & 1ull);  // half of the dropped range, ties to even
  u &= ~drop;
  float f = (float)__longlong_as_double((long long)u);  // exact, or +-inf on overflow
  return (bf16_t)(__float_as_uint(f) >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
  static __device__ __forceinline__ float from_d(double x) { return (float)x; }  // RNE
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float to_f(bf16_t x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ bf16_t from_f(float x) { return f32_to_bf16(x); }
  static __device__ __forceinline__ bf16_t from_d(double x) { return f64_to_bf16_rne(x); }
};

// ------------------------------------------------------------ MFMA fragments
// 16x16 tiles, wave64.  Operand fragment for "k-chunk of 32": lane l holds row
// (or column) l%16 and the 8 k-values 8*(l/16) .. 8*(l/16)+7.  The output
// fragment holds rows 4*(l/16)+i (i = 0..3) of column l%16.
struct FragBF16 { bf16x8 v; };
struct FragF32 { float v[8]; };

template <typename T> struct Frag32;
template <> struct Frag32<bf16_t> { typedef FragBF16 type; };
template <> struct Frag32<float> { typedef FragF32 type; };

__device__ __forceinline__ f32x4 mma_k32(const FragBF16& a, const FragBF16& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
// Float32 operands: eight 16x16x4 steps, step j taking slot j of every lane.
__device__ __forceinline__ f32x4 mma_k32(const FragF32& a, const FragF32& b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}

// Load 8 consecutive elements as an operand fragment.
__device__ __forceinline__ void load_frag(FragBF16& f, const bf16_t* p) {
  f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}
__device__ __forceinline__ void load_frag(FragF32& f, const float* p) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Indexer operand: 16-dim vectors, lane l holds row l%16 dims 4*(l/16)..+3.
struct IdxFragBF16 { short4v v; };
struct IdxFragF32 { float v[4]; };
template <typename T> struct IdxFrag;
template <> struct IdxFrag<bf16_t> { typedef IdxFragBF16 type; };
template <> struct IdxFrag<float> { typedef IdxFragF32 type; };

__device__ __forceinline__ void load_idx_frag(IdxFragBF16& f, const bf16_t* p) {
  f.v = __builtin_bit_cast(short4v, *reinterpret_cast<const uint2*>(p));
}
__device__ __forceinline__ void load_idx_frag(IdxFragF32& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
}

// Raw indexer dot products q_idx . k_idx for a 16 (keys) x 16 (queries) tile:
// A = index keys, B = index queries.  Every kernel that needs an indexer score
// goes through this one function, so a given (key, query) pair always gets the
// same float32 value.
__device__ __forceinline__ f32x4 idx_dot_tile(const IdxFragBF16& kf, const IdxFragBF16& qf) {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(kf.v, qf.v, z, 0, 0, 0);
}
__device__ __forceinline__ f32x4 idx_dot_tile(const IdxFragF32& kf, const IdxFragF32& qf) {
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(kf.v[j], qf.v[j], c, 0, 0, 0);
  return c;
}

// A value the optimiser must treat as unknown (an empty asm statement that
// claims to modify the register): keeps it from turning per-tile expressions
// into per-element loop counters that each cost a register and an add.
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The indexer score s = (q_idx . k_idx) / sqrt(16); the scale is exact.
__device__ __forceinline__ float idx_score(float dot) { return dot * 0.25f; }

// ------------------------------------------------------------ reductions
// Data-parallel-primitive moves within a row of 16 lanes (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Sum over each row of 16 lanes, identical in all 16 lanes: a butterfly over
// lane pairs (xor 1, xor 2 via quad permutes, then the half-row and row mirrors),
// so every lane adds the same pairs in the same order.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of a 16x16 MFMA
// output tile), the same value in all four.  gfx950's row and half-wave swaps run on
// the VALU (a shuffle through ds_bpermute takes the LDS pipe, an index computation and
// a wait for every outstanding LDS read).  Each swap leaves x[l] in one result and
// x[l ^ 16] (or x[l ^ 32]) in the other, so max and + see the same pairs as an xor
// butterfly and give the same bits.  All 64 lanes must be active.
__device__ __forceinline__ float col4_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col4_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ------------------------------------------------------------ register-only wave scans
// DPP moves of the GFX9 family, 32 bits at a time (64-bit values move as two halves):
// row_shr:n (0x110 + n) moves a value n lanes up inside each 16-lane row, lanes with no
// source reading 0; row_bcast:15 (0x142) adds lane 15's value into the next row, and
// row_bcast:31 (0x143) lane 31's into rows 2 and 3 (rows outside the row mask read 0).
// None of them touches LDS or needs lane-index arithmetic.  Every helper below reads
// other lanes' registers, so it must be called with all 64 lanes of the wave active
// (uniform control flow), as every caller in this library does.
template <int CTRL, int ROWS, bool BC, typename V>
__device__ __forceinline__ V dppv(V x) {
  if constexpr (sizeof(V) == 4) {
    return __builtin_bit_cast(V, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, BC));
  } else {
    static_assert(sizeof(V) == 8, "32- or 64-bit values");
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWS, 0xF, BC);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWS, 0xF, BC);
    return __builtin_bit_cast(V, ((unsigned long long)hi << 32) | lo);
  }
}
// Inclusive sum over lanes 0..l of a wave (all 64 lanes active): a Hillis-Steele scan
// inside each row, then the row totals carried up by the two broadcasts.
template <typename V>
__device__ __forceinline__ V wave_scan_add(V x) {
  x += dppv<0x111, 0xF, true>(x);
  x += dppv<0x112, 0xF, true>(x);
  x += dppv<0x114, 0xF, true>(x);
  x += dppv<0x118, 0xF, true>(x);
  x += dppv<0x142, 0xA, false>(x);
  x += dppv<0x143, 0xC, false>(x);
  return x;
}
// The partner values of a row swap (lane l ^ 16) or half-wave swap (lane l ^ 32): op is
// applied to the swap's two results, which hold x[l] and its partner in either order.
template <bool HALF, typename V, typename Op>
__device__ __forceinline__ V swap_op(V x, Op op) {
  if constexpr (sizeof(V) == 4) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = HALF ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                        : __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__builtin_bit_cast(V, (uint32_t)a[0]), __builtin_bit_cast(V, (uint32_t)a[1]));
  } else {
    const unsigned long long u = __builtin_bit_cast(unsigned long long, x);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const auto a = HALF ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = HALF ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const V v0 = __builtin_bit_cast(V, ((unsigned long long)(uint32_t)b[0] << 32) | (uint32_t)a[0]);
    const V v1 = __builtin_bit_cast(V, ((unsigned long long)(uint32_t)b[1] << 32) | (uint32_t)a[1]);
    return op(v0, v1);
  }
}
// op over all 64 lanes, the same value in every lane: quad swaps, half-row and row
// mirrors, then the row and half-wave swaps.  Every lane combines the same pairs, so a
// commutative op (max, or a float sum) gives identical bits in all lanes.
// (Within a row this is the xor 1, 2, 4, 8 butterfly: after the two quad steps all lanes
// of a quad hold the same value, so the mirrors pair the same values as xor 4 and xor 8.)
template <typename V, typename Op>
__device__ __forceinline__ V row16_allreduce(V x, Op op) {
  x = op(x, dppv<0xB1, 0xF, false>(x));    // quad_perm [1,0,3,2]
  x = op(x, dppv<0x4E, 0xF, false>(x));    // quad_perm [2,3,0,1]
  x = op(x, dppv<0x141, 0xF, false>(x));   // row_half_mirror
  return op(x, dppv<0x140, 0xF, false>(x));   // row_mirror
}
template <typename V, typename Op>
__device__ __forceinline__ V wave_allreduce(V x, Op op) {
  x = row16_allreduce(x, op);
  x = swap_op<false>(x, op);
  return swap_op<true>(x, op);
}
// op over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one column of a 16x16 MFMA tile)
template <typename V, typename Op>
__device__ __forceinline__ V col4_op(V x, Op op) {
  return swap_op<true>(swap_op<false>(x, op), op);
}
struct OpAdd { template <typename V> __device__ __forceinline__ V operator()(V a, V b) const { return a + b; } };
struct OpMax { template <typename V> __device__ __forceinline__ V operator()(V a, V b) const { return a > b ? a : b; } };

struct OpFmax { __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); } };
// max / sum over the 64 lanes of a wave, the same value in every lane (register-only)
__device__ __forceinline__ float wave_max(float x) { return wave_allreduce(x, OpFmax()); }
__device__ __forceinline__ float wave_sum(float x) { return wave_allreduce(x, OpAdd()); }

}  // namespace rtp
