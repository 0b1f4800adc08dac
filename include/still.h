/*
 * still.h -- C ABI of the STILL intra-layer hybrid attention operator on
 * AMD Instinct MI355X (gfx950).
 *
 * The operator comes from "STILL: Selecting Tokens for Intra-Layer Hybrid
 * Attention to Linearize LLMs" (Meng et al., 2026).  Section references are
 * to the paper's full-text web page; figure captions are from its list view.
 *
 * For every attention layer it
 *   1. runs sliding-window softmax attention and scores every token's
 *      Self-Saliency inside its window (Sec. 3.1, Fig. 2);
 *   2. keeps the top-`topk` tokens of every complete chunk of `chunk` tokens,
 *      decided once per chunk (delayed selection, Sec. 3.3), separately per
 *      KV head (Sec. 3.3: routing is per head);
 *   3. runs softmax attention over the selected tokens and linear attention
 *      with the Norm-Preserved Feature Map (NP-Map, Sec. 3.2) over every other
 *      token that has left the window (Sec. 3.3, Appendix A.2);
 *   4. merges both branches with one shared normaliser (Fig. 2, "hybrid
 *      aggregation").
 *
 * Where the pages leave a step open this library follows these readings:
 *   - Score_t = sum_j a_j ln((a_j+eps)/(a~_j+eps)) over token t's own window
 *     row a (itself included) and its leave-one-out row a~ (a~_t = 0)
 *     (Appendix A.3, Lemma 1 and Remark);
 *   - a KV head routes by the mean score of its query heads;
 *   - top-k ties go to the lower position;
 *   - token j is routed for query t once j <= t - window; chunk decisions are
 *     therefore complete in time only when window >= chunk (Appendix A.7.5:
 *     the window spans one chunk);
 *   - phi(x) = [softmax(z); softmax(-z)], z = ||x|| P x / ||P x||;
 *   - the gate W_g (list view Table 9; full text Sec. 4.1, App. A.6.1) is a
 *     weight gamma = sigmoid(g) per token and query head on the linear
 *     branch, whose logits g = x W_g the caller computes like q, k, v;
 *   - out = (sum_SA e^{tau q.k} v + gamma sum_LA phi_q.phi_k v) /
 *           (sum_SA e^{tau q.k}   + gamma sum_LA phi_q.phi_k).
 *
 * Conventions for every call
 *   - Tensors are dense row-major, innermost dimension last, on the current
 *     HIP device, 16-byte aligned.  q / out: [B, N, Hq, d]; k / v:
 *     [B, N, Hkv, d]; query head h reads KV head h / (Hq / Hkv).
 *   - `dtype` is the element type of q, k, v, out and the cached K/V:
 *     STILL_BF16 (bf16 storage, fp32 arithmetic, results rounded to nearest
 *     even) or STILL_F32.  NP-Map projections, scores and linear states are
 *     always fp32.
 *   - The caller owns and allocates every buffer (inputs, outputs, workspace,
 *     cache).  The library never allocates, frees or synchronises: work is
 *     enqueued on `stream` and results are valid once the stream reaches
 *     that point.  No state survives a call except a per-process cache of
 *     device properties, so calls on distinct buffers are thread-safe.
 *   - Every entry point validates all arguments on the host before
 *     launching anything, returns a still_status, and never aborts.
 *   - gate_opt (every compute call): gate logits g [B, N, Hq] fp32 (N = 1 for
 *     a decode step), 4-byte aligned, read only; NULL means no gate
 *     (gamma = 1, the operator without the component).  gamma = 0 leaves
 *     window + selected softmax attention.
 */
#ifndef STILL_H
#define STILL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STILL_ABI_VERSION 6

typedef enum {
    STILL_OK = 0,
    STILL_ERR_INVALID_ARG = -1,  /* null/misaligned pointer, bad shape or parameter   */
    STILL_ERR_UNSUPPORTED = -2,  /* valid for the method, not built here (e.g. d=96)  */
    STILL_ERR_WORKSPACE = -3,    /* workspace_bytes smaller than the size call asks   */
    STILL_ERR_CAPACITY = -4,     /* the selected-token cache could overflow           */
    STILL_ERR_HIP = -5           /* a kernel launch failed (hipGetLastError)          */
} still_status;

typedef enum { STILL_F32 = 0, STILL_BF16 = 1 } still_dtype;

/* Force the general kernels even where the gfx950 MFMA kernels apply
 * (cross-checking; both compute the same operator). */
#define STILL_FLAG_GENERAL_KERNELS 1u
/* Routing criterion, in bits 1-3 of flags (shifted by STILL_ROUTE_SHIFT):
 * the per-chunk top-k ranks tokens by the Self-Saliency score (Sec. 3.1,
 * default) or by one of the criteria the pages compare it with under the same
 * routing and cache settings (full text Sec. 4 ablation, Table 7):
 *   DIAGONAL  the token's own weight a_tt in its window row, mean over the
 *             group's query heads
 *   QK        its own logit tau q_t.k_t, mean over the group's query heads
 *   KEYNORM   ||k_t||
 *   UNIFORM   lambda tokens evenly spaced in each chunk (offsets floor(i C/lambda))
 *   RANDOM    lambda tokens drawn uniformly per chunk: score = top 24 bits of
 *             splitmix64(((b * Hkv + g) << 32) | t) times 2^-24
 * Scores returned by the forward and kept in the decode cache are the
 * criterion's values. */
#define STILL_ROUTE_SHIFT 1
#define STILL_ROUTE_MASK (7u << STILL_ROUTE_SHIFT)
#define STILL_ROUTE_SALIENCY 0u
#define STILL_ROUTE_DIAGONAL 1u
#define STILL_ROUTE_QK 2u
#define STILL_ROUTE_KEYNORM 3u
#define STILL_ROUTE_UNIFORM 4u
#define STILL_ROUTE_RANDOM 5u

/* Problem statement (Sec. 3.3 and Appendix A.4: window W, chunk C, per-chunk
 * quota lambda; Sec. 3.2: NP-Map feature size d').
 *   batch B >= 0, seqlen N >= 0 (1 for a decode step),
 *   n_q_heads Hq >= 1, n_kv_heads Hkv >= 1 with Hq % Hkv == 0,
 *   head_dim d in {64, 128}, feat_dim d' == d,
 *   window W >= 0, chunk C in [1, 1024], topk lambda >= 0 (clamped to C),
 *   W == 0 requires lambda == 0; lambda > 0 requires W >= C,
 *   eps > 0 (Self-Saliency smoothing, Appendix A.3),
 *   softmax_scale tau > 0, or 0 for 1/sqrt(d). */
typedef struct {
    int32_t batch, seqlen, n_q_heads, n_kv_heads, head_dim, feat_dim;
    int32_t window, chunk, topk;
    float eps, softmax_scale;
    int32_t dtype;   /* still_dtype */
    uint32_t flags;  /* STILL_FLAG_* */
} still_shape;

/* Decode cache of Sec. 3.3 "Recurrent Form": the sliding window, the
 * permanently retained selected tokens, and the linear-attention state of
 * every other token that has left the window.  All device memory, all owned
 * by the caller; layouts per (sequence b, KV head g):
 *   win_k, win_v   [B, Hkv, W, d]  dtype; position p lives in slot p % W
 *   win_route      [B, Hkv, W]     u8: 0 pending, 1 selected (SA), 2 linear (LA)
 *   pend_score     [B, Hkv, C]     fp32 group-mean scores of the open chunk,
 *                                  position p in slot p % C
 *   sel_k, sel_v   [B, Hkv, cap, d] dtype, selected tokens in the order they
 *                                  left the window (ascending position)
 *   sel_count      [B, Hkv]        int32 rows of sel_k/sel_v in use
 *   lin_S          [B, Hkv, d', d] fp32, sum of phi_k(k_j) v_j^T (Appendix A.2)
 *   lin_z          [B, Hkv, d']    fp32, sum of phi_k(k_j)
 *   pos            next position t (host value, shared by the batch; the
 *                  decode step advances it by one on success).
 * Pointers of parts that a shape does not use (window parts when W == 0,
 * selected parts when lambda == 0) may be NULL. */
typedef struct {
    void* win_k;
    void* win_v;
    uint8_t* win_route;
    float* pend_score;
    void* sel_k;
    void* sel_v;
    int32_t* sel_count;
    int32_t sel_cap;
    float* lin_S;
    float* lin_z;
    int64_t pos;
} still_cache;

/* Version of this header's ABI (STILL_ABI_VERSION). */
int32_t still_abi_version(void);

/* Static text for a still_status value. */
const char* still_status_str(int status);

/* Certified per-chunk quota of Appendix A.4:
 * lambda = floor((m - W) / ceil(n_max / C)), so that every length up to n_max
 * keeps at most m tokens (window included) in the softmax cache.  Returns -1
 * for m < W, C < 1 or n_max < 1. */
int32_t still_topk_for_budget(int32_t m, int32_t window, int32_t chunk, int64_t n_max);

/* Bytes of device workspace still_hybrid_attn_fwd needs for `shape`.
 * Returns STILL_OK and writes *bytes, or an error status for an invalid
 * shape. */
int still_fwd_workspace_size(const still_shape* shape, size_t* bytes);

/* Chunk-parallel forward (Sec. 3.3, "Chunk-Wise Parallel Form"): the whole
 * sequence at once, causal, with the same routing as the recurrent form.
 *   q, k, v         inputs (layouts above), read only
 *   wphi_q, wphi_k  [Hkv, d'/2, d] fp32 NP-Map projections of queries and
 *                   keys (Sec. 3.2), one pair per KV head
 *   out             [B, N, Hq, d] dtype, written
 *   scores_opt      [B, Hkv, N] fp32 group-mean Self-Saliency, or NULL
 *   sel_idx_opt     [B, Hkv, N / C, min(topk, C)] int32 selected positions of
 *                   every complete chunk, ascending, or NULL
 *   stats_opt       [B, N, Hq, 4] fp32, 16-byte aligned, or NULL: per query
 *                   head (m, l, 0, c), the reference point of the shared
 *                   normaliser (natural-log units), the normaliser at that
 *                   reference (softmax and linear weights together, Fig. 2
 *                   hybrid aggregation), 0, and c = exp(-m) / l for a query
 *                   with linear terms (0 otherwise); with the output, what
 *                   still_hybrid_attn_bwd can start from instead of
 *                   recomputing them
 *   cache_opt       if not NULL, filled as the recurrent form would leave it
 *                   after these N tokens (prefill -> decode hand-off):
 *                   cache_opt->pos must equal N on entry; needs
 *                   sel_cap >= min(topk,C) * ceil(max(0, N - W) / C)
 *                   (else STILL_ERR_CAPACITY)
 *   workspace       >= still_fwd_workspace_size bytes of device memory
 * N == 0 or B == 0 is a no-op returning STILL_OK once the shape is valid (no
 * pointer is inspected). */
int still_hybrid_attn_fwd(const still_shape* shape, const void* q, const void* k, const void* v,
                          const float* wphi_q, const float* wphi_k, const float* gate_opt,
                          void* out, float* scores_opt,
                          int32_t* sel_idx_opt, float* stats_opt, still_cache* cache_opt, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace one decode step needs for `shape` (seqlen is
 * ignored) and a selected cache of `sel_cap` rows. */
int still_decode_workspace_size(const still_shape* shape, int32_t sel_cap, size_t* bytes);

/* One recurrent step (Sec. 3.3, "Recurrent Form") at position t = cache->pos
 * for all B sequences:
 *   1. the token at t - W leaves the window: if its chunk selected it, it is
 *      appended to sel_k/sel_v for good; otherwise it is folded into
 *      lin_S / lin_z (W == 0: the new token itself goes to the linear state);
 *   2. k_t, v_t enter the window;
 *   3. the Self-Saliency of t (mean over the group's query heads) is stored
 *      in pend_score;
 *   4. out = hybrid attention of q_t over window + selected tokens + linear
 *      state;
 *   5. when t closes a chunk, its top-k tokens are marked selected, the rest
 *      linear.
 *   q [B, 1, Hq, d], k / v [B, 1, Hkv, d], out [B, 1, Hq, d].
 * Returns STILL_ERR_CAPACITY (nothing launched) when
 * min(topk,C) * ceil((t + 1 - W) / C) > sel_cap.  On STILL_OK cache->pos is
 * incremented. */
int still_hybrid_attn_decode_step(const still_shape* shape, const void* q, const void* k,
                                  const void* v, const float* wphi_q, const float* wphi_k,
                                  const float* gate_opt, still_cache* cache, void* out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Serving form of the decode step: the same step (1-5 above) with one
 * position per sequence, for a batch whose sequences have different lengths
 * (each sequence's cache filled by its own forward, or by earlier steps).
 *   pos_dev   [B] int64 device memory, 8-byte aligned: the next position t_b
 *             of sequence b; read by the step's kernels and advanced by one
 *             (on the stream) by its last kernel
 *   max_pos   host value >= every t_b, used for the capacity check
 *             min(topk,C) * ceil((max_pos + 1 - W) / C) <= sel_cap
 *   cache->pos is neither read nor written.
 * Chunk-end selection (step 5) happens per sequence, when t_b closes a chunk
 * of sequence b.  Errors as for still_hybrid_attn_decode_step; a NULL or
 * misaligned pos_dev or a negative max_pos is STILL_ERR_INVALID_ARG.  (The
 * serving setting of Sec. 4.6: every request decodes at its own length.) */
int still_hybrid_attn_decode_step_ragged(const still_shape* shape, const void* q, const void* k,
                                         const void* v, const float* wphi_q, const float* wphi_k,
                                         const float* gate_opt, still_cache* cache, int64_t* pos_dev,
                                         int64_t max_pos,
                                         void* out, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* Size of the device scratch that still_hybrid_attn_decode_step_noalloc
 * keeps per GPU (32 MiB: a batch of 64 Llama-3-8B-shaped sequences, 32 / 8
 * heads, d = 128, with selected caches of up to about 24K rows per KV head). */
#define STILL_DECODE_SCRATCH_BYTES ((size_t)32 << 20)

/* still_hybrid_attn_decode_step without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (less the
 * workspace), same computation, same validation and errors as
 * still_hybrid_attn_decode_step.  Its kernels use a scratch array that the
 * library holds in device memory instead: STILL_DECODE_SCRATCH_BYTES on each
 * GPU the library runs on, reserved with the library's device code on that
 * GPU and kept until the process ends.  A step that needs more scratch than
 * that (still_decode_workspace_size reports the need) returns
 * STILL_ERR_WORKSPACE before anything is launched.  The call allocates no
 * memory and calls no allocating routine.  Every call on one GPU uses that
 * GPU's one scratch array: calls whose work can overlap on the same GPU
 * (unordered streams, several threads) race and give undefined results;
 * calls ordered on one stream are safe.  Nothing in the scratch needs
 * clearing: every byte a step reads is written earlier in the same step.
 * The first call on a GPU looks up the array's device address there (with
 * that GPU current); a failed lookup returns STILL_ERR_HIP. */
int still_hybrid_attn_decode_step_noalloc(const still_shape* shape, const void* q, const void* k,
                                          const void* v, const float* wphi_q,
                                          const float* wphi_k, const float* gate_opt,
                                          still_cache* cache, void* out, hipStream_t stream);

/* Bytes of device workspace still_hybrid_attn_bwd needs for `shape`. */
int still_bwd_workspace_size(const still_shape* shape, size_t* bytes);

/* Backward pass of still_hybrid_attn_fwd: gradients of
 * L = sum(dout * out) with respect to q, k, v and the two NP-Map
 * projections, for the training the paper's linearization runs through the
 * chunk-wise parallel form (Sec. 3.3; Sec. 4.1 "Experimental Setups",
 * training strategy; App. A.6.1).  The routing is held fixed: the selection
 * is a constant mask, so nothing flows through the scores or the top-k, and
 * M = max(0, max logit) cancels between numerator and denominator.  Where
 * an NP-Map projection P x is zero the map is taken as locally constant
 * (zero gradient).
 *   q, k, v, wphi_q, wphi_k  as given to the forward, read only
 *   sel_idx   [B, Hkv, N / C, min(topk, C)] int32, the forward's sel_idx
 *             output (the routing to differentiate under); entries outside
 *             their chunk, and repeats, are ignored.  May be NULL when
 *             min(topk, C) == 0 or N < C.
 *   dout      [B, N, Hq, d] dtype, the gradient of L w.r.t. out
 *   out_opt, stats_opt  the forward's out and stats_opt for the same inputs,
 *             gate and routing, both or neither (else STILL_ERR_INVALID_ARG),
 *             16-byte aligned: the matrix-core path then takes each query's
 *             reference, normaliser and linear weight from stats_opt and
 *             dout . out from out instead of a first pass that recomputes
 *             them; the fp32 kernels ignore them
 *   fwd_workspace_opt, fwd_workspace_bytes  if not NULL, the workspace of the
 *             forward call that produced sel_idx (same shape and inputs,
 *             untouched since): the matrix-core path then reads the keys'
 *             NP-Map features and the linear prefixes the forward left there
 *             instead of recomputing them (STILL_ERR_WORKSPACE when smaller
 *             than still_fwd_workspace_size); the fp32 kernels ignore it
 *   dq        [B, N, Hq, d] fp32, written
 *   dk, dv    [B, N, Hkv, d] fp32, written
 *   dwphi_q, dwphi_k  [Hkv, d'/2, d] fp32, written
 *   dgate_opt [B, N, Hq] fp32: the gradient w.r.t. the gate logits, written
 *             when gate_opt is given and this is not NULL; ignored without
 *             a gate
 *   workspace >= still_bwd_workspace_size bytes of device memory
 * For bf16 storage with d = d' = 128, window 64 / 128 / 256, chunk 64 / 128 /
 * 256 no longer than the window, and 1, 2, 4 or 8 query heads per KV head,
 * every term runs on the matrix cores: a first pass (the forward's main
 * kernel over compact lists of the given selection; skipped when out_opt and
 * stats_opt are given) gives each query's reference, normaliser and
 * dout . out; the softmax terms are formed from
 * bf16 logit and dout . v products with dS rounded to bf16, as the forward
 * rounds its probabilities, and the linear terms, the NP-Map backward and
 * the projection gradients take bf16 operands too (gradients to about 1e-2
 * relative); every other shape uses fp32 kernels (about 1e-6).
 * STILL_FLAG_GENERAL_KERNELS
 * forces the fp32 kernels everywhere; the routing-criterion flags do not
 * matter.  N == 0
 * or B == 0 writes zeros to dwphi_q and dwphi_k (when not NULL) and nothing
 * else.  Errors as for the forward; a missing sel_idx where it is needed is
 * STILL_ERR_INVALID_ARG. */
int still_hybrid_attn_bwd(const still_shape* shape, const void* q, const void* k, const void* v,
                          const float* wphi_q, const float* wphi_k, const float* gate_opt,
                          const int32_t* sel_idx, const void* dout, const void* out_opt,
                          const float* stats_opt, const void* fwd_workspace_opt,
                          size_t fwd_workspace_bytes, float* dq, float* dk,
                          float* dv, float* dwphi_q, float* dwphi_k, float* dgate_opt,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace still_future_kv_utility needs for `shape`. */
int still_future_kv_utility_workspace_size(const still_shape* shape, size_t* bytes);

/* Future-KV-utility diagnostic (full text App. A.7.4, Table 12): how much
 * full causal attention each remote key receives from the queries after its
 * window,
 *   util[b, g, j] = sum over the query heads h of KV head g and the queries
 *                   t >= j + W of softmax over j' <= t of (tau q_t,h . k_j')
 * (plain causal softmax attention: nothing is routed).  Keys with no query
 * after their window (j > N - 1 - W) get 0.  Ranking the eligible keys
 * j <= N - 1 - W by util and comparing the top ones with the tokens a
 * routing criterion selected measures how well a causal local score
 * predicts future use.
 *   q [B, N, Hq, d], k [B, N, Hkv, d] dtype, read only; util [B, Hkv, N]
 *   fp32, written.  Only batch, seqlen, heads, head_dim, window, eps,
 *   softmax_scale and dtype of the shape matter; it must still be valid.
 * N == 0 or B == 0 is a no-op.  Errors as for the forward. */
int still_future_kv_utility(const still_shape* shape, const void* q, const void* k, float* util,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Instrumented forms of the entry points, for measurement (they compute
 * exactly what the plain calls compute).  Before the i-th kernel launch the
 * call records events[i] on `stream`, and events[n] after the last launch,
 * so hipEventElapsedTime(events[i], events[i+1]) is launch i's duration on
 * that stream.  kernel_names_opt[i] (if not NULL) receives a static name of
 * launch i.  *n_launches receives n.  Needs max_events >= n + 1, else
 * STILL_ERR_INVALID_ARG before anything is launched; events are created and
 * destroyed by the caller. */
#define STILL_MAX_LAUNCHES 24
int still_hybrid_attn_fwd_timed(const still_shape* shape, const void* q, const void* k,
                                const void* v, const float* wphi_q, const float* wphi_k,
                                const float* gate_opt, void* out, float* scores_opt, int32_t* sel_idx_opt,
                                float* stats_opt, still_cache* cache_opt, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                int32_t max_events, int32_t* n_launches, const char** kernel_names_opt);
int still_hybrid_attn_decode_step_timed(const still_shape* shape, const void* q, const void* k,
                                        const void* v, const float* wphi_q,
                                        const float* wphi_k, const float* gate_opt,
                                        still_cache* cache, void* out,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream, hipEvent_t* events,
                                        int32_t max_events, int32_t* n_launches,
                                        const char** kernel_names_opt);
int still_hybrid_attn_bwd_timed(const still_shape* shape, const void* q, const void* k,
                                const void* v, const float* wphi_q, const float* wphi_k,
                                const float* gate_opt, const int32_t* sel_idx, const void* dout,
                                const void* out_opt, const float* stats_opt,
                                const void* fwd_workspace_opt, size_t fwd_workspace_bytes,
                                float* dq, float* dk, float* dv, float* dwphi_q, float* dwphi_k,
                                float* dgate_opt, void* workspace,
                                size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                                int32_t max_events, int32_t* n_launches,
                                const char** kernel_names_opt);

#ifdef __cplusplus
}
#endif
#endif /* STILL_H */
