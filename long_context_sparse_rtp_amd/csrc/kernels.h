// Internal interface between the C ABI layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/rtp.h"

namespace rtp {

// Problem description passed by value to every kernel.
struct ProbDev {
  int batch, Hq, Hkv, R, n_sink, window, n_local;
  int max_q, max_k;
  int64_t Tq, Tk;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t kcap;                    // rows per sequence in the key arrays (0: packed at cu_k offsets)
  int ring;                        // key rows of a sequence form a ring of n_sink + window slots
  int ret_heads[RTP_MAX_HEADS];    // slot -> query head
  int local_heads[RTP_MAX_HEADS];  // local index -> query head
  // local heads grouped by KV head, at most attn_decode_tile_heads() per tile: tile t covers
  // local_heads[ltile_start[t] .. ltile_start[t] + ltile_cnt[t])
  int n_ltiles;
  int ltile_start[RTP_MAX_HEADS];
  int ltile_cnt[RTP_MAX_HEADS];
  // the same grouping with up to attn_decode_group_heads() heads per tile (the
  // bfloat16 decode path scores a tile's heads together on the matrix cores)
  int n_gtiles;
  int gtile_start[RTP_MAX_HEADS];
  int gtile_cnt[RTP_MAX_HEADS];
  // retrieval slots grouped by KV head the same way (slots r .. r + cnt - 1 of one
  // group); max_rtile = the largest tile
  int n_rtiles, max_rtile;
  uint8_t rtile_start[RTP_MAX_HEADS];
  uint8_t rtile_cnt[RTP_MAX_HEADS];
};
static_assert(sizeof(ProbDev) <= 3584, "ProbDev travels as a kernel argument (4 KB in all)");

__host__ __device__ inline int kv_of(const ProbDev& p, int h) { return (h * p.Hkv) / p.Hq; }

// First row of sequence b in k, v, k_pre, k_idx and the LIST idx: the packed
// offset cu_k[b], or b * capacity in the per-sequence capacity layout.
__device__ __forceinline__ int key_row0(const ProbDev& p, int b) {
  return p.kcap > 0 ? (int)((int64_t)b * p.kcap) : p.cu_k[b];
}
// Row of position n within its sequence: n itself, or its slot in a ring that
// keeps the n_sink sinks and the last `window` positions.
__device__ __forceinline__ int key_slot(const ProbDev& p, int n) {
  if (!p.ring || n < p.n_sink) return n;
  return p.n_sink + (n - p.n_sink) % p.window;
}

// Workspace layouts (bytes), shared by rtp_workspace_size and the launchers.
size_t ws_select_decode(const ProbDev& p);
int select_decode_max_keys();   // longest sequence LIST selection accepts
size_t ws_select_prefill(const ProbDev& p);
size_t ws_attn_decode(const ProbDev& p, int mode);  // mode 0: retrieval heads, 1: local heads
int attn_decode_max_rows();   // (head, sequence) rows one decode attention call accepts
int attn_decode_tile_heads(); // local heads of one KV group handled together in decode
int attn_decode_group_heads(); // local heads of one KV group per tile of the bfloat16 decode path

hipError_t launch_index_keys(const ProbDev& p, bool bf16, const void* k_pre, const float* w_k,
                             void* k_idx, hipStream_t s);
// new tokens [total_new] at the end of every sequence: K/V rows and their index keys
hipError_t launch_append_kv(const ProbDev& p, bool bf16, const int32_t* cu_new, int64_t total_new,
                            const void* k_new, const void* v_new, const void* k_pre_new, const float* w_k,
                            void* k, void* v, void* k_idx, hipStream_t s);
// top_k == nullptr: dynamic top-p over top_p[batch]; otherwise fixed top-k over top_k[batch]
hipError_t launch_select_decode(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                const void* k_idx, const float* top_p, const int32_t* top_k,
                                const rtp_selection& sel, void* ws, hipStream_t s);
hipError_t launch_select_prefill(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                 const void* k_idx, const float* top_p, const int32_t* top_k,
                                 const rtp_selection& sel, void* ws, hipStream_t s);
// the pages' block-granular top-p (decode, LIST output)
size_t ws_select_blocks(const ProbDev& p);
hipError_t launch_select_blocks(const ProbDev& p, bool bf16, const void* q_pre, const float* w_q,
                                const void* k_idx, const float* top_p, const rtp_selection& sel, void* ws,
                                hipStream_t s);
// mode 0: retrieval heads over sel LIST; mode 1: local heads over window + sinks
// The library's own scratch for callers that cannot allocate: a file-scope device
// array of decode_scratch_bytes() bytes.  decode_scratch() returns its address on
// the current device (resolved once per device, on that device's first call).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** out);
hipError_t launch_attn_decode(const ProbDev& p, bool bf16, int mode, const void* q, const void* k,
                              const void* v, const rtp_selection* sel, void* out, float* lse,
                              void* ws, hipStream_t s);
// mode 0: retrieval heads with THRESHOLD membership; mode 1: local heads
hipError_t launch_attn_prefill(const ProbDev& p, bool bf16, int mode, const void* q, const void* k,
                               const void* v, const void* k_idx, const rtp_selection* sel,
                               void* out, float* lse, hipStream_t s);

}  // namespace rtp
