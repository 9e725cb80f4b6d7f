/*
 * rtp.h - C ABI of the RTPurbo-style sparse-attention hot path for AMD MI355X (gfx950).
 *
 * The method (page "Full Attention Strikes Back: Transferring Full Attention
 * into Sparse within Hundred Training Steps", paper-graph-ui summary of
 * arXiv 2605.16928, section 3.4) splits the query heads of a GQA attention
 * layer in two:
 *   - retrieval heads keep the whole KV cache; each query scores every cached
 *     key through a 16-dim pre-RoPE indexer, keeps the smallest highest-score
 *     set whose softmax mass reaches top-p, and runs exact softmax attention
 *     (head_dim 128, post-RoPE q and k) over that set only;
 *   - local heads attend to the first n_sink tokens plus a causal sliding
 *     window.
 *
 * Layouts (packed varlen, token-major, row-major, no padding):
 *   q, out            [T_q, Hq, 128]   dtype
 *   k, v, k_pre       [T_k, Hkv, 128]  dtype
 *   q_pre             [T_q, R, 128]    dtype   (pre-RoPE q of the R retrieval heads)
 *   w_q, w_k          [R, 16, 128]     float32 (indexer projections, one per retrieval head)
 *   k_idx, q_idx      [R, T_k | T_q, 16] dtype (index keys / queries)
 *   lse               [Hq, T_q]        float32 (natural log; optional)
 * Sequence b owns key rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) and query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]); query i of sequence b sits at position
 * L_k(b) - L_q(b) + i.  Prefill therefore has L_q = L_k; decode has L_q = 1 and
 * the current token's K/V already appended.  Query head h reads KV head
 * floor(h * Hkv / Hq) (contiguous GQA groups).  Retrieval slot r is query head
 * ret_heads[r].
 *
 * Ownership and execution: every pointer marked (dev) is device memory owned by
 * the caller.  The library allocates nothing, never synchronises, keeps no
 * pointer after a call returns, and keeps no state between calls except a
 * per-thread error string and, for rtp_sparse_attn_decode_noalloc, the device
 * address of its static scratch on each device.  All work is enqueued on the caller's HIP stream
 * (NULL = default stream); buffers must stay alive until that stream has run it.
 *
 * Errors: every argument check runs on the host before any launch, so a call
 * either enqueues all its work or changes nothing.  A launch failure returns
 * RTP_ERR_HIP; rtp_last_hip_error() gives the HIP message.  Device pointers
 * must be non-NULL (unless marked optional) and 16-byte aligned.  Inputs must
 * be finite; NaN or Inf gives undefined output (never out-of-bounds access).
 */
#ifndef RTP_H
#define RTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define RTP_API __attribute__((visibility("default")))
#else
#define RTP_API
#endif

typedef enum {
  RTP_OK = 0,
  RTP_ERR_INVALID_ARG = 1,
  RTP_ERR_UNSUPPORTED = 2,
  RTP_ERR_WORKSPACE_TOO_SMALL = 3,
  RTP_ERR_HIP = 4
} rtp_status;

typedef enum { RTP_F32 = 0, RTP_BF16 = 1 } rtp_dtype;

typedef enum { RTP_SEL_LIST = 0, RTP_SEL_THRESHOLD = 1 } rtp_sel_mode;

/* Which call a workspace size is asked for. */
typedef enum {
  RTP_CALL_SELECT = 1,
  RTP_CALL_SPARSE_PREFILL = 2,
  RTP_CALL_SPARSE_DECODE = 3,
  RTP_CALL_LOCAL = 4,
  RTP_CALL_SELECT_BLOCKS = 5
} rtp_call;

#define RTP_MAX_HEADS 128

/* Problem description (a host struct). */
typedef struct {
  int32_t batch;                 /* number of sequences, >= 1 */
  int32_t n_q_heads;             /* Hq, 1..RTP_MAX_HEADS */
  int32_t n_kv_heads;            /* Hkv, divides Hq */
  int32_t head_dim;              /* must be 128 */
  int32_t idx_dim;               /* must be 16 */
  int32_t n_ret;                 /* R = number of retrieval heads, 0..Hq */
  const int32_t *ret_heads;      /* host [R]: distinct, ascending query-head ids */
  int32_t n_sink;                /* local heads: leading sink tokens, >= 0 (the paper uses 4) */
  int32_t window;                /* local heads: window length W >= 1 (keys pos-W < n <= pos) */
  rtp_dtype dtype;               /* q, k, v, q_pre, k_pre, out, k_idx, q_idx */
  const int32_t *cu_seqlens_q;   /* (dev) [batch+1] */
  const int32_t *cu_seqlens_k;   /* (dev) [batch+1] */
  int32_t max_seqlen_q;          /* host: max_b L_q(b) (grid sizing; L_q(b) <= L_k(b)) */
  int32_t max_seqlen_k;          /* host: max_b L_k(b) */
  int64_t total_q;               /* host: T_q = cu_seqlens_q[batch] */
  int64_t total_k;               /* host: rows of the key arrays: cu_seqlens_k[batch] when packed,
                                    batch * k_capacity otherwise */
  int64_t k_capacity;            /* 0: packed keys (sequence b at rows cu_seqlens_k[b] ..);
                                    > 0: sequence b at rows [b * k_capacity, b * k_capacity + L_k(b)),
                                    so a cache grows in place (L_k(b) <= k_capacity) */
  int32_t ring;                  /* 1: the key rows of a sequence are a ring that keeps only what
                                    local heads read: position n < n_sink at row n, any later
                                    position at row n_sink + (n - n_sink) % window; requires
                                    k_capacity = n_sink + window, n_ret = 0 and one query per
                                    sequence (rtp_local_attn, rtp_append_kv).  0: plain rows. */
} rtp_problem;

/* Output of rtp_select_topp, input of the sparse attention calls (device pointers). */
typedef struct {
  void *q_idx;       /* (dev) [R, T_q, 16] dtype: rounded indexer queries, written by select */
  float *tau;        /* (dev) THRESHOLD: [R, T_q] score threshold (-inf when p >= 1) */
  int32_t *tie_pos;  /* (dev) THRESHOLD: [R, T_q] last admitted position among scores == tau
                        (INT32_MAX: all of them) */
  int32_t *count;    /* (dev) [R, T_q] size of the selected set */
  int32_t *idx;      /* (dev) LIST: [R, T_k]; slot (r, b) starts at r*T_k + cu_seqlens_k[b] */
} rtp_selection;

/*
 * Key layouts.  k, v, k_pre and k_idx rows of sequence b start at cu_seqlens_k[b]
 * (packed) or at b * k_capacity (capacity layout); the LIST slice (r, b) of
 * sel->idx starts at r * total_k + that row.  Lengths always come from
 * cu_seqlens_k[b + 1] - cu_seqlens_k[b].  A ring (ring = 1) holds the n_sink
 * sinks and the last `window` positions of each sequence in n_sink + window
 * rows: the storage local heads need, since they never read anything else (page
 * "Full Attention Strikes Back ...", section 3.4 "Local Head Attention Pattern").
 */

/* Bytes of workspace a call needs for this problem (0 = none).  Pure host function. */
RTP_API size_t rtp_workspace_size(const rtp_problem *prob, rtp_call call, rtp_sel_mode mode);

/*
 * rtp_index_keys: the 16-dim index-key cache of every retrieval head.
 *   k_idx[r, n, :] = RNE_dtype( W^K_r . k_pre[n, kv(ret_heads[r]), :] )
 * Low-dimensional projection of the pre-RoPE key (section 3.4 "Low-Dimensional
 * Projection Mechanism and Stage-1 Training", score-computation equation; the
 * paragraph on the 16-dimensional scoring cost keeps these projected keys
 * cached once computed).  The dot product is accumulated in
 * float64 and rounded once to dtype (round to nearest even).
 *   k_pre (dev) [T_k, Hkv, 128] dtype;  w_k (dev) [R, 16, 128] float32;
 *   k_idx (dev, out) [R, T_k, 16] dtype.
 */
RTP_API rtp_status rtp_index_keys(const rtp_problem *prob, const void *k_pre, const float *w_k,
                          void *k_idx, void *stream);

/*
 * rtp_append_kv: append new tokens to the caches of every sequence (one per
 * sequence in a decode step; a whole prompt to fill a ring after prefill).
 * New token t of sequence b (t = 0 .. n_b - 1, n_b = cu_seqlens_new[b+1] -
 * cu_seqlens_new[b]) takes position L_k(b) - n_b + t, where L_k(b) from prob is
 * the length after the append; its K and V rows (all KV heads) go to that
 * position's row of k and v, and every retrieval slot r gets
 *   k_idx[r, row, :] = RNE_dtype(W^K_r . k_pre_new[t, kv(ret_heads[r]), :])
 * computed exactly as rtp_index_keys computes it (the index keys are kept
 * once computed, section 3.4, paragraph on the 16-dimensional scoring cost).
 * In a ring, new tokens that are neither sinks nor among the last `window`
 * positions are skipped.
 *   cu_seqlens_new (dev) [batch+1]; total_new (host) = cu_seqlens_new[batch];
 *   k_new, v_new, k_pre_new (dev) [total_new, Hkv, 128] dtype; w_k (dev) [R,16,128];
 *   k, v (dev, in/out) key arrays in the layout of prob; k_idx (dev, in/out)
 *   [R, total_k, 16].  k_pre_new, w_k and k_idx may be NULL when n_ret = 0.
 */
RTP_API rtp_status rtp_append_kv(const rtp_problem *prob, const int32_t *cu_seqlens_new, int64_t total_new,
                         const void *k_new, const void *v_new, const void *k_pre_new, const float *w_k,
                         void *k, void *v, void *k_idx, void *stream);

/*
 * rtp_select_topp: indexer scores and dynamic top-p per (retrieval head, query).
 *   q_idx = RNE_dtype(W^Q_r . q_pre)  (written to sel->q_idx)
 *   s_n   = (q_idx . k_idx_n) / sqrt(16) for every key n <= pos (float32)
 *   S     = smallest set of keys, taken by descending s (ties: ascending
 *           position), whose softmax(s) mass reaches top_p[b]; p >= 1 keeps all.
 * Section 3.4 "Dynamic Top-p Selection Mechanism", Eq. 5.  The selection is
 * token-exact (not the pages' 64-token block approximation).
 *   q_pre (dev) [T_q, R, 128]; w_q (dev) [R, 16, 128] float32;
 *   k_idx (dev) [R, T_k, 16] dtype (from rtp_index_keys);
 *   top_p (dev) [batch] float32.
 *   mode LIST (decode; requires max_seqlen_q == 1, else RTP_ERR_UNSUPPORTED):
 *     writes sel->idx (ascending key positions, within the sequence) and sel->count.
 *   mode THRESHOLD (any L_q): writes sel->tau, sel->tie_pos, sel->count with
 *     S = {n <= pos : s_n > tau} U {n <= pos : s_n == tau and n <= tie_pos};
 *     tie_pos = INT32_MAX when no token scoring exactly tau is left out.
 *   sel->q_idx is always written.  ws: rtp_workspace_size(prob, RTP_CALL_SELECT, mode) bytes.
 */
RTP_API rtp_status rtp_select_topp(const rtp_problem *prob, const void *q_pre, const float *w_q,
                           const void *k_idx, const float *top_p, rtp_sel_mode mode,
                           const rtp_selection *sel, void *ws, size_t ws_bytes, void *stream);

/*
 * rtp_select_topk: the same indexer scores with a fixed budget instead of top-p -
 * the static top-k (k = 4096 on the page) that the page measures dynamic top-p
 * against (sections "Evaluation Methodology", baselines, and "Ablation Studies
 * and Robustness Checks", static top-k vs. dynamic top-p).
 *   S = the min(k, L) keys n <= pos with the highest s_n, equal scores taken by
 *       ascending position; k = top_k[b], values below 1 read as 1.
 *   top_k (dev) [batch] int32.  Every other argument, the output (LIST or
 *   THRESHOLD, same encoding: tau is the k-th highest score, -inf when every
 *   key is kept) and the workspace (RTP_CALL_SELECT) are those of rtp_select_topp,
 *   so the sparse attention calls consume either selection unchanged.
 */
RTP_API rtp_status rtp_select_topk(const rtp_problem *prob, const void *q_pre, const float *w_q,
                           const void *k_idx, const int32_t *top_k, rtp_sel_mode mode,
                           const rtp_selection *sel, void *ws, size_t ws_bytes, void *stream);

/*
 * rtp_select_topp_blocks: the pages' own block-granular approximation of top-p
 * for decode (section "Hardware-Aware Fast Top-p Decoding Kernel", the
 * sort-free histogram, steps 1-5).  The same indexer scores as rtp_select_topp;
 * then, per (retrieval head, sequence):
 *   - keys are cut into 64-token blocks from position 0 (the last may be short);
 *     block b keeps m_b = max score and its mass sum_{n in b} exp(s_n - max s);
 *   - [min m_b, max m_b] is cut into 256 equal bins, each block's mass goes to
 *     the bin of its m_b (all blocks in the top bin when every m_b is equal);
 *   - bins are scanned from the top to the first where the cumulative mass
 *     reaches top_p[b] of the total (p >= 1: every block);
 *   - every block in that bin or above is kept whole.
 * Output is LIST only (requires max_seqlen_q == 1, else RTP_ERR_UNSUPPORTED):
 * sel->idx holds the kept blocks' positions ascending, sel->count their number;
 * sel->tau (optional) the lower edge of the crossing bin in score units (-inf
 * when every block is kept), sel->tie_pos (optional) INT32_MAX.  sel->q_idx is
 * written.  ws: rtp_workspace_size(prob, RTP_CALL_SELECT_BLOCKS, RTP_SEL_LIST).
 */
RTP_API rtp_status rtp_select_topp_blocks(const rtp_problem *prob, const void *q_pre, const float *w_q,
                                  const void *k_idx, const float *top_p, const rtp_selection *sel,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * rtp_sparse_attn_prefill: exact attention of every retrieval-head query over its
 * THRESHOLD set, O = sum_{n in S} softmax_S(q . k_n / sqrt(128)) v_n
 * (section 3.4, equation after Eq. 5), float32 accumulation.  Membership is
 * recomputed from sel->q_idx and k_idx with the same arithmetic rtp_select_topp
 * used, so the set is exactly the one selected.
 *   q (dev) [T_q, Hq, 128]; k, v (dev) [T_k, Hkv, 128]; k_idx (dev) [R, T_k, 16];
 *   sel: THRESHOLD output of rtp_select_topp;  out (dev) [T_q, Hq, 128]: only the
 *   retrieval heads' rows are written;  lse (dev, optional) [Hq, T_q].
 */
RTP_API rtp_status rtp_sparse_attn_prefill(const rtp_problem *prob, const void *q, const void *k,
                                   const void *v, const void *k_idx, const rtp_selection *sel,
                                   void *out, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * rtp_sparse_attn_decode: the same attention for one query per sequence over the
 * LIST set (sel->idx / sel->count), split over the list with a log-sum-exp merge.
 * Requires max_seqlen_q == 1.  ws: rtp_workspace_size(prob, RTP_CALL_SPARSE_DECODE, LIST).
 */
RTP_API rtp_status rtp_sparse_attn_decode(const rtp_problem *prob, const void *q, const void *k,
                                  const void *v, const rtp_selection *sel, void *out, float *lse,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * rtp_sparse_attn_decode_noalloc: rtp_sparse_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, result and kernels, but no
 * workspace argument: the split partials live in the library's own static device
 * scratch of RTP_NOALLOC_SCRATCH_BYTES bytes (one copy per device, held until the
 * process ends, its address resolved on the first call on each device).  The call
 * allocates and frees nothing.  A problem whose decode workspace,
 * rtp_workspace_size(prob, RTP_CALL_SPARSE_DECODE, RTP_SEL_LIST), exceeds the
 * scratch is rejected before any launch with RTP_ERR_WORKSPACE_TOO_SMALL
 * (rtp_last_hip_error() then names both sizes).  Every call on one device shares
 * that scratch: calls that overlap on a device (concurrent streams, or host
 * threads enqueueing to different streams) race; calls on one stream are ordered
 * by it and are safe.  Nothing in the scratch needs clearing between calls.
 */
#define RTP_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
RTP_API rtp_status rtp_sparse_attn_decode_noalloc(const rtp_problem *prob, const void *q, const void *k,
                                          const void *v, const rtp_selection *sel, void *out, float *lse,
                                          void *stream);

/*
 * rtp_local_attn: every non-retrieval head attends to keys
 *   {n <= pos : pos - W < n} U {n < min(n_sink, pos + 1)}
 * with dense softmax (section 3.4 "Local Head Attention Pattern").  Prefill-shaped
 * and decode-shaped problems are both accepted.  Writes only the local heads'
 * rows of out / lse.  ws: rtp_workspace_size(prob, RTP_CALL_LOCAL, 0).
 */
RTP_API rtp_status rtp_local_attn(const rtp_problem *prob, const void *q, const void *k, const void *v,
                          void *out, float *lse, void *ws, size_t ws_bytes, void *stream);

RTP_API const char *rtp_status_str(rtp_status s);
RTP_API const char *rtp_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RTP_H */
