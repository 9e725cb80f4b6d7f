// C ABI of the sparse-attention hot path: argument validation (host only, before
// any launch) and dispatch to the kernel launchers.  See include/rtp.h for the
// contract of every entry point.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kernels.h"

using rtp::ProbDev;

namespace {

thread_local char g_err[256] = "";

void set_hip_error(hipError_t e) {
  snprintf(g_err, sizeof(g_err), "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

rtp_status check_problem(const rtp_problem* pr, ProbDev* out) {
  if (!pr) return RTP_ERR_INVALID_ARG;
  if (pr->batch < 1) return RTP_ERR_INVALID_ARG;
  if (pr->n_q_heads < 1 || pr->n_q_heads > RTP_MAX_HEADS) return RTP_ERR_INVALID_ARG;
  if (pr->n_kv_heads < 1 || pr->n_q_heads % pr->n_kv_heads != 0) return RTP_ERR_INVALID_ARG;
  if (pr->head_dim != 128 || pr->idx_dim != 16) return RTP_ERR_UNSUPPORTED;
  if (pr->n_ret < 0 || pr->n_ret > pr->n_q_heads) return RTP_ERR_INVALID_ARG;
  if (pr->n_ret > 0 && !pr->ret_heads) return RTP_ERR_INVALID_ARG;
  for (int r = 0; r < pr->n_ret; ++r) {
    const int h = pr->ret_heads[r];
    if (h < 0 || h >= pr->n_q_heads) return RTP_ERR_INVALID_ARG;
    if (r > 0 && h <= pr->ret_heads[r - 1]) return RTP_ERR_INVALID_ARG;  // distinct, ascending
  }
  if (pr->n_sink < 0 || pr->window < 1) return RTP_ERR_INVALID_ARG;
  if (pr->n_sink > 64) return RTP_ERR_UNSUPPORTED;  // sinks must fit the first 64-key tile
  if (pr->dtype != RTP_F32 && pr->dtype != RTP_BF16) return RTP_ERR_INVALID_ARG;
  if (!aligned4(pr->cu_seqlens_q) || !aligned4(pr->cu_seqlens_k)) return RTP_ERR_INVALID_ARG;
  if (pr->max_seqlen_q < 1 || pr->max_seqlen_k < 1) return RTP_ERR_INVALID_ARG;
  if (pr->max_seqlen_q > pr->max_seqlen_k) return RTP_ERR_INVALID_ARG;
  if (pr->total_q < 1 || pr->total_k < 1) return RTP_ERR_INVALID_ARG;
  if (pr->total_q > (int64_t)pr->batch * pr->max_seqlen_q) return RTP_ERR_INVALID_ARG;
  if (pr->k_capacity == 0 && pr->total_k > (int64_t)pr->batch * pr->max_seqlen_k) return RTP_ERR_INVALID_ARG;
  if (pr->total_q >= INT32_MAX || pr->total_k >= INT32_MAX) return RTP_ERR_UNSUPPORTED;
  // key layout: packed, per-sequence capacity, or a ring of sinks + window
  if (pr->k_capacity < 0 || (pr->ring != 0 && pr->ring != 1)) return RTP_ERR_INVALID_ARG;
  if (pr->ring && pr->k_capacity != (int64_t)pr->n_sink + pr->window) return RTP_ERR_INVALID_ARG;
  if (pr->k_capacity > 0) {
    if (pr->total_k != (int64_t)pr->batch * pr->k_capacity) return RTP_ERR_INVALID_ARG;
    if (!pr->ring && pr->max_seqlen_k > pr->k_capacity) return RTP_ERR_INVALID_ARG;
  }
  if (pr->ring && (pr->n_ret != 0 || pr->max_seqlen_q != 1)) return RTP_ERR_UNSUPPORTED;
  if (out) {
    ProbDev& p = *out;
    memset(&p, 0, sizeof(p));
    p.batch = pr->batch;
    p.Hq = pr->n_q_heads;
    p.Hkv = pr->n_kv_heads;
    p.R = pr->n_ret;
    p.n_sink = pr->n_sink;
    p.window = pr->window;
    p.max_q = pr->max_seqlen_q;
    p.max_k = pr->max_seqlen_k;
    p.Tq = pr->total_q;
    p.Tk = pr->total_k;
    p.cu_q = pr->cu_seqlens_q;
    p.cu_k = pr->cu_seqlens_k;
    p.kcap = pr->k_capacity;
    p.ring = pr->ring;
    bool is_ret[RTP_MAX_HEADS] = {false};
    for (int r = 0; r < p.R; ++r) {
      p.ret_heads[r] = pr->ret_heads[r];
      is_ret[pr->ret_heads[r]] = true;
    }
    p.n_local = 0;
    for (int h = 0; h < p.Hq; ++h)
      if (!is_ret[h]) p.local_heads[p.n_local++] = h;
    // local heads in runs of one KV group, at most `cap` per tile (heads ascend, so a
    // group's local heads are consecutive)
    auto tiles = [&](int cap, int& n, int* start, int* cnt) {
      n = 0;
      for (int i = 0; i < p.n_local; ++i) {
        const int t = n - 1;
        if (t >= 0 && cnt[t] < cap && rtp::kv_of(p, p.local_heads[start[t]]) == rtp::kv_of(p, p.local_heads[i])) {
          ++cnt[t];
        } else {
          start[n] = i;
          cnt[n] = 1;
          ++n;
        }
      }
    };
    tiles(rtp::attn_decode_tile_heads(), p.n_ltiles, p.ltile_start, p.ltile_cnt);
    tiles(rtp::attn_decode_group_heads(), p.n_gtiles, p.gtile_start, p.gtile_cnt);
    // retrieval slots (ascending heads: a group's slots are consecutive)
    p.n_rtiles = 0;
    p.max_rtile = 0;
    for (int r = 0; r < p.R; ++r) {
      const int t = p.n_rtiles - 1;
      if (t >= 0 && p.rtile_cnt[t] < rtp::attn_decode_group_heads() &&
          rtp::kv_of(p, p.ret_heads[p.rtile_start[t]]) == rtp::kv_of(p, p.ret_heads[r])) {
        ++p.rtile_cnt[t];
      } else {
        p.rtile_start[p.n_rtiles] = (uint8_t)r;
        p.rtile_cnt[p.n_rtiles] = 1;
        ++p.n_rtiles;
      }
    }
    for (int t = 0; t < p.n_rtiles; ++t) p.max_rtile = p.max_rtile > p.rtile_cnt[t] ? p.max_rtile : p.rtile_cnt[t];
  }
  return RTP_OK;
}

rtp_status finish(hipError_t e) {
  if (e != hipSuccess) {
    set_hip_error(e);
    return RTP_ERR_HIP;
  }
  return RTP_OK;
}

size_t ws_need(const ProbDev& p, rtp_call call, rtp_sel_mode mode) {
  switch (call) {
    case RTP_CALL_SELECT:
      return mode == RTP_SEL_LIST ? rtp::ws_select_decode(p) : rtp::ws_select_prefill(p);
    case RTP_CALL_SPARSE_PREFILL:
      return 0;
    case RTP_CALL_SPARSE_DECODE:
      return rtp::ws_attn_decode(p, 0);
    case RTP_CALL_LOCAL:
      return p.max_q == 1 ? rtp::ws_attn_decode(p, 1) : 0;
    case RTP_CALL_SELECT_BLOCKS:
      return rtp::ws_select_blocks(p);
  }
  return 0;
}

rtp_status check_ws(const ProbDev& p, rtp_call call, rtp_sel_mode mode, const void* ws, size_t ws_bytes) {
  const size_t need = ws_need(p, call, mode);
  if (need == 0) return RTP_OK;
  if (ws_bytes < need) return RTP_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(ws)) return RTP_ERR_INVALID_ARG;
  return RTP_OK;
}

// Shared by rtp_select_topp (top_k == nullptr) and rtp_select_topk (top_p == nullptr).
rtp_status select_common(const rtp_problem* prob, const void* q_pre, const float* w_q, const void* k_idx,
                         const float* top_p, const int32_t* top_k, rtp_sel_mode mode, const rtp_selection* sel,
                         void* ws, size_t ws_bytes, void* stream) {
  ProbDev p;
  rtp_status st = check_problem(prob, &p);
  if (st != RTP_OK) return st;
  if (mode != RTP_SEL_LIST && mode != RTP_SEL_THRESHOLD) return RTP_ERR_INVALID_ARG;
  if (p.R == 0) return RTP_OK;
  if (!sel || !aligned16(q_pre) || !aligned16(w_q) || !aligned16(k_idx) || !aligned4(top_k ? (const void*)top_k : top_p))
    return RTP_ERR_INVALID_ARG;
  if (!aligned16(sel->q_idx) || !aligned4(sel->count)) return RTP_ERR_INVALID_ARG;
  if (mode == RTP_SEL_LIST) {
    if (p.max_q != 1 || p.Tq != p.batch) return RTP_ERR_UNSUPPORTED;
    if (p.max_k > rtp::select_decode_max_keys()) return RTP_ERR_UNSUPPORTED;
    if (!aligned4(sel->idx)) return RTP_ERR_INVALID_ARG;
    if ((sel->tau && !aligned4(sel->tau)) || (sel->tie_pos && !aligned4(sel->tie_pos))) return RTP_ERR_INVALID_ARG;
  } else {
    if (!aligned4(sel->tau) || !aligned4(sel->tie_pos)) return RTP_ERR_INVALID_ARG;
  }
  st = check_ws(p, RTP_CALL_SELECT, mode, ws, ws_bytes);
  if (st != RTP_OK) return st;
  const bool bf16 = prob->dtype == RTP_BF16;
  hipStream_t s = (hipStream_t)stream;
  if (mode == RTP_SEL_LIST)
    return finish(rtp::launch_select_decode(p, bf16, q_pre, w_q, k_idx, top_p, top_k, *sel, ws, s));
  return finish(rtp::launch_select_prefill(p, bf16, q_pre, w_q, k_idx, top_p, top_k, *sel, ws, s));
}

// Argument checks shared by rtp_sparse_attn_decode and its no-alloc variant.
rtp_status check_sparse_decode(const rtp_problem* prob, ProbDev* p, const void* q, const void* k, const void* v,
                               const rtp_selection* sel, const void* out, const float* lse) {
  rtp_status st = check_problem(prob, p);
  if (st != RTP_OK) return st;
  if (p->max_q != 1 || p->Tq != p->batch) return RTP_ERR_UNSUPPORTED;
  if (p->R == 0) return RTP_OK;
  if ((int64_t)p->R * p->batch > rtp::attn_decode_max_rows()) return RTP_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RTP_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return RTP_ERR_INVALID_ARG;
  if (!sel || !aligned4(sel->idx) || !aligned4(sel->count)) return RTP_ERR_INVALID_ARG;
  return RTP_OK;
}

}  // namespace

extern "C" {

size_t rtp_workspace_size(const rtp_problem* prob, rtp_call call, rtp_sel_mode mode) {
  ProbDev p;
  if (check_problem(prob, &p) != RTP_OK) return 0;
  return ws_need(p, call, mode);
}

rtp_status rtp_append_kv(const rtp_problem* prob, const int32_t* cu_seqlens_new, int64_t total_new,
                         const void* k_new, const void* v_new, const void* k_pre_new, const float* w_k, void* k,
                         void* v, void* k_idx, void* stream) {
  ProbDev p;
  rtp_status st = check_problem(prob, &p);
  if (st != RTP_OK) return st;
  // a ring takes a whole prompt (most of it skipped); other layouts have a row per new token
  if (total_new < 0 || total_new >= INT32_MAX || (!p.ring && total_new > p.Tk)) return RTP_ERR_INVALID_ARG;
  if (total_new == 0) return RTP_OK;
  if (!aligned4(cu_seqlens_new) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k) || !aligned16(v))
    return RTP_ERR_INVALID_ARG;
  if (p.R > 0 && (!aligned16(k_pre_new) || !aligned16(w_k) || !aligned16(k_idx))) return RTP_ERR_INVALID_ARG;
  return finish(rtp::launch_append_kv(p, prob->dtype == RTP_BF16, cu_seqlens_new, total_new, k_new, v_new,
                                      k_pre_new, w_k, k, v, k_idx, (hipStream_t)stream));
}

rtp_status rtp_index_keys(const rtp_problem* prob, const void* k_pre, const float* w_k, void* k_idx,
                          void* stream) {
  ProbDev p;
  rtp_status st = check_problem(prob, &p);
  if (st != RTP_OK) return st;
  if (p.R == 0) return RTP_OK;
  if (!aligned16(k_pre) || !aligned16(w_k) || !aligned16(k_idx)) return RTP_ERR_INVALID_ARG;
  return finish(rtp::launch_index_keys(p, prob->dtype == RTP_BF16, k_pre, w_k, k_idx, (hipStream_t)stream));
}

rtp_status rtp_select_topp(const rtp_problem* prob, const void* q_pre, const float* w_q, const void* k_idx,
                           const float* top_p, rtp_sel_mode mode, const rtp_selection* sel, void* ws,
                           size_t ws_bytes, void* stream) {
  return select_common(prob, q_pre, w_q, k_idx, top_p, nullptr, mode, sel, ws, ws_bytes, stream);
}

rtp_status rtp_select_topk(const rtp_problem* prob, const void* q_pre, const float* w_q, const void* k_idx,
                           const int32_t* top_k, rtp_sel_mode mode, const rtp_selection* sel, void* ws,
                           size_t ws_bytes, void* stream) {
  return select_common(prob, q_pre, w_q, k_idx, nullptr, top_k, mode, sel, ws, ws_bytes, stream);
}

rtp_status rtp_select_topp_blocks(const rtp_problem* prob, const void* q_pre, const float* w_q, const void* k_idx,
                                  const float* top_p, const rtp_selection* sel, void* ws, size_t ws_bytes,
                                  void* stream) {
  ProbDev p;
  rtp_status st = check_problem(prob, &p);
  if (st != RTP_OK) return st;
  if (p.R == 0) return RTP_OK;
  if (!sel || !aligned16(q_pre) || !aligned16(w_q) || !aligned16(k_idx) || !aligned4(top_p))
    return RTP_ERR_INVALID_ARG;
  if (!aligned16(sel->q_idx) || !aligned4(sel->count) || !aligned4(sel->idx)) return RTP_ERR_INVALID_ARG;
  if ((sel->tau && !aligned4(sel->tau)) || (sel->tie_pos && !aligned4(sel->tie_pos))) return RTP_ERR_INVALID_ARG;
  if (p.max_q != 1 || p.Tq != p.batch) return RTP_ERR_UNSUPPORTED;
  if (p.max_k > rtp::select_decode_max_keys()) return RTP_ERR_UNSUPPORTED;
  st = check_ws(p, RTP_CALL_SELECT_BLOCKS, RTP_SEL_LIST, ws, ws_bytes);
  if (st != RTP_OK) return st;
  return finish(rtp::launch_select_blocks(p, prob->dtype == RTP_BF16, q_pre, w_q, k_idx, top_p, *sel, ws,
                                          (hipStream_t)stream));
}

rtp_status rtp_sparse_attn_prefill(const rtp_problem* prob, const void* q, const void* k, const void* v,
                                   const void* k_idx, const rtp_selection* sel, void* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  ProbDev p;
  rtp_status st = check_problem(prob, &p);
  if (st != RTP_OK) return st;
  if (p.R == 0) return RTP_OK;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_idx) || !aligned16(out))
    return RTP_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return RTP_ERR_INVALID_ARG;
  if (!sel || !aligned16(sel->q_idx) || !aligned4(sel->tau) || !aligned4(sel->tie_pos))
    return RTP_ERR_INVALID_ARG;
  return finish(rtp::launch_attn_prefill(p, prob->dtype == RTP_BF16, 0, q, k, v, k_idx, sel, out, lse,
                                         (hipStream_t)stream));
}


rtp_status rtp_sparse_attn_decode(const rtp_problem* prob, const void* q, const void* k, const void* v,
                                  const rtp_selection* sel, void* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  ProbDev p;
  rtp_status st = check_sparse_decode(prob, &p, q, k, v, sel, out, lse);
  if (st != RTP_OK || p.R == 0) return st;
  st = check_ws(p, RTP_CALL_SPARSE_DECODE, RTP_SEL_LIST, ws, ws_bytes);
  if (st != RTP_OK) return st;
  return finish(rtp::launch_attn_decode(p, prob->dtype == RTP_BF16, 0, q, k, v, sel, out, lse, ws,
                                        (hipStream_t)stream));
}

rtp_status rtp_sparse_attn_decode_noalloc(const rtp_problem* prob, const void* q, const void* k, const void* v,
                                          const rtp_selection* sel, void* out, float* lse, void* stream) {
  ProbDev p;
  rtp_status st = check_sparse_decode(prob, &p, q, k, v, sel, out, lse);
  if (st != RTP_OK || p.R == 0) return st;
  const size_t need = ws_need(p, RTP_CALL_SPARSE_DECODE, RTP_SEL_LIST);
  if (need > rtp::decode_scratch_bytes()) {
    snprintf(g_err, sizeof(g_err), "rtp_sparse_attn_decode_noalloc: the problem needs %zu bytes of scratch, "
             "the library's static scratch holds %zu", need, rtp::decode_scratch_bytes());
    return RTP_ERR_WORKSPACE_TOO_SMALL;
  }
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = rtp::decode_scratch(&ws);
    if (e != hipSuccess) return finish(e);
  }
  return finish(rtp::launch_attn_decode(p, prob->dtype == RTP_BF16, 0, q, k, v, sel, out, lse, ws,
                                        (hipStream_t)stream));
}

rtp_status rtp_local_attn(const rtp_problem* prob, const void* q, const void* k, const void* v, void* out,
                          float* lse, void* ws, size_t ws_bytes, void* stream) {
  ProbDev p;
  rtp_status st = check_problem(prob, &p);
  if (st != RTP_OK) return st;
  if (p.n_local == 0) return RTP_OK;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return RTP_ERR_INVALID_ARG;
  if (lse && !aligned4(lse)) return RTP_ERR_INVALID_ARG;
  const bool bf16 = prob->dtype == RTP_BF16;
  hipStream_t s = (hipStream_t)stream;
  if (p.max_q == 1) {
    if (p.Tq != p.batch) return RTP_ERR_INVALID_ARG;
    if ((int64_t)p.n_ltiles * p.batch > rtp::attn_decode_max_rows()) return RTP_ERR_UNSUPPORTED;
    st = check_ws(p, RTP_CALL_LOCAL, RTP_SEL_LIST, ws, ws_bytes);
    if (st != RTP_OK) return st;
    return finish(rtp::launch_attn_decode(p, bf16, 1, q, k, v, nullptr, out, lse, ws, s));
  }
  if (p.ring) return RTP_ERR_UNSUPPORTED;
  return finish(rtp::launch_attn_prefill(p, bf16, 1, q, k, v, nullptr, nullptr, out, lse, s));
}

const char* rtp_status_str(rtp_status s) {
  switch (s) {
    case RTP_OK: return "ok";
    case RTP_ERR_INVALID_ARG: return "invalid argument";
    case RTP_ERR_UNSUPPORTED: return "unsupported problem";
    case RTP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case RTP_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* rtp_last_hip_error(void) { return g_err; }

}  // extern "C"
