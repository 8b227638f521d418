/*
 * rtp.h -- C ABI of the head-wise sparse attention library (RTPurbo hot path)
 * for AMD Instinct MI355X (gfx950).
 *
 * Method: "Full Attention Strikes Back: Transferring Full Attention into Sparse
 * within Hundred Training Steps" (arXiv 2605.16928).  Its abstract (OpenAlex
 * record and podcast episode page) and the atlas.scime.ai research-map summary
 * describe it in prose only:
 *   - a small subset of attention heads ("retrieval heads") keep the full KV
 *     cache; the others ("local heads") attend to a few sink tokens plus a
 *     sliding window (abstract, observation (1); summary, "Approach");
 *   - retrieval heads pick tokens with a 16-dimensional pre-RoPE indexer and a
 *     query-adaptive top-p threshold over the indexer's softmax mass (abstract,
 *     observations (2) and (3); summary, "Approach"), then attend over the
 *     gathered K/V of that set only (abstract: a small indexer picks the tokens
 *     that sparse attention reads);
 *   - during prefill retrieval heads stay dense (summary, "Limitations").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor pointers are DEVICE pointers into caller-owned memory, contiguous
 *    in the layouts written next to each argument, 16-byte aligned.  bf16 means
 *    IEEE bfloat16 raw bits (uint16_t); results are rounded to nearest even.
 *  - Ownership: the library allocates nothing.  Scratch space comes from the
 *    caller's workspace `ws` of `ws_bytes` bytes (256-byte aligned); size it with
 *    rtp_workspace_bytes().  rtp_topp_select and rtp_decode_step keep radix
 *    histograms, counters and per-range records in their workspace that their
 *    kernels reset themselves: such a workspace must be ZERO-FILLED before its
 *    first use, every call that completes leaves that region zero again, and it
 *    must not be handed to another kind of call in between.  (The exception is
 *    the selection region's last part, the digit tables of ranges with many
 *    distinct candidates, B * Hq_r * ceil(n_cap / RTP_SEL_RANGE) * 2 KiB rounded
 *    up to 256 bytes: a call writes a table whole before it reads it, and leaves
 *    the tables as they are.)  The region depends
 *    on the descriptor only (not on n_ctx), so one workspace serves a growing
 *    context.  The other calls need no particular content.  A workspace may be
 *    reused by later calls on the same stream; calls that run concurrently need
 *    distinct workspaces.  After a device fault, zero-fill it again before reuse.
 *  - Errors: every argument is validated on the host before anything is
 *    enqueued.  On error nothing is launched and no output is touched; the
 *    status is returned and rtp_last_error() (thread-local) explains it.
 *    RTP_OK means the work was enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream).  There is no implicit synchronisation and no host<->device
 *    copy; counts and thresholds stay on the device.  RTP_EDEVICE reports a
 *    failed launch; faults inside kernels surface at the caller's next sync.
 *    Fault injection: when the environment variable RTP_FAULT_INJECT is set to a
 *    non-empty value, every call that passes its host checks returns RTP_EDEVICE
 *    ("injected device failure") where it would first touch the device, with
 *    nothing enqueued, so callers can test their device-error paths on a host
 *    without a GPU.
 *  - Tracing: with the environment variable RTP_ROCTX set to a non-empty value at
 *    the first call, every call that enqueues work is wrapped in a roctx range
 *    named after it (visible with rocprofv3 --marker-trace).
 *  - Heads: G = n_q_heads / n_kv_heads; KV head g serves query heads
 *    g*G .. g*G+G-1.  Retrieval KV heads (kv_role[g] == 1) are numbered by rank
 *    r = 0,1,.. in increasing g; retrieval query head g*G+t has the compact index
 *    r*G + t, which indexes w_q_idx, scores, row stats and selected sets.
 *  - Supported: head_dim 64 or 128; G in {1,2,4,8}; idx_dim in {4,8,16,32};
 *    n_cap < 2^30; batch >= 1 (prefill: batch == 1).  I below = idx_dim.
 */
#ifndef RTP_H
#define RTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rtp_status {
  RTP_OK = 0,
  RTP_EINVAL = 1,        /* bad argument: null pointer, bad size, bad value, misaligned */
  RTP_EUNSUPPORTED = 2,  /* valid but not implemented: head_dim, group size, idx_dim */
  RTP_EWORKSPACE = 3,    /* ws_bytes smaller than rtp_workspace_bytes() */
  RTP_EDEVICE = 4        /* a HIP launch or runtime call failed */
} rtp_status;

/* One attention layer.  Everything here lives in HOST memory. */
typedef struct rtp_layer_desc {
  int32_t batch;          /* sequences in the batch (B) */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;       /* D */
  int32_t idx_dim;        /* indexer dimension: 16 on the pages' design (abstract, observation
                             (2)); 4, 8 and 32 for the ablation (summary, "Surprising
                             findings"); 32 needs G <= 4; rtp_decode_step needs 16 */
  int64_t n_cap;          /* cache capacity = token stride of every per-token tensor */
  const uint8_t* kv_role; /* [Hkv] HOST array: 1 = retrieval head, 0 = local head */
  int32_t n_sinks;        /* local heads: sink tokens at the start of the sequence (>= 0) */
  int32_t window;         /* local heads: sliding window, counting the query token (>= 1) */
  int32_t kv_layout;      /* RTP_KV_FULL or RTP_KV_COMPACT (decode calls; see below) */
} rtp_layer_desc;

/*
 * K/V cache layouts of the decode calls (the cache pointer each call takes):
 *  RTP_KV_FULL     every head: [B][Hkv][n_cap][D], token j at row j.
 *  RTP_KV_COMPACT  only retrieval heads keep their whole history, local heads keep
 *                  their sinks and window (abstract: the full KV cache is retained for
 *                  retrieval heads only; summary, "Approach"):
 *                    retrieval cache [B][Hkv_r][n_cap][D], token j at row j;
 *                    local ring      [B][Hkv_l][n_sinks + window][D], token j at row
 *                    j if j < n_sinks, else n_sinks + (j - n_sinks) % window.
 *                  rtp_sparse_decode_attn takes the retrieval cache, rtp_window_sink_attn
 *                  the ring; rtp_append_token writes both.  Prefill needs RTP_KV_FULL.
 */
#define RTP_KV_FULL 0
#define RTP_KV_COMPACT 1

/* Token-index range of one entry of a selected-set range index (sel_starts). */
#define RTP_SEL_RANGE 1024

/* Which call rtp_workspace_bytes() sizes. */
typedef enum rtp_call {
  RTP_CALL_INDEXER_SCORE = 0,
  RTP_CALL_TOPP_SELECT = 1,
  RTP_CALL_SPARSE_DECODE = 2,
  RTP_CALL_WINDOW_SINK = 3,
  RTP_CALL_PREFILL = 4,
  RTP_CALL_DECODE_STEP = 5
} rtp_call;

/* Workspace bytes that call `which` needs for this layer at context n_ctx
 * (prefill: n_ctx = chunk rows C).  Returns 0 for an invalid descriptor. */
size_t rtp_workspace_bytes(const rtp_layer_desc* desc, int64_t n_ctx, int which);

/*
 * rtp_indexer_score -- indexer scores of every cached token for every retrieval
 * query head, plus the softmax statistics of each score row.
 * (abstract, observation (2); summary, "Approach": 16-dim pre-RoPE projection)
 *
 *   q_idx[b,c]   = q_pre[b, h(c)] . W_q_idx[c]            (fp32, never rounded)
 *   s[b,c,j]     = idx_scale * <q_idx[b,c], k_idx[b, r(c), j]>   for 0 <= j < n_ctx
 *   row_max[b,c] = max_j s[b,c,j];   row_sum[b,c] = sum_j exp(s[b,c,j] - row_max[b,c])
 *
 *   q_pre   bf16 [B][Hq][D]         pre-RoPE queries (all heads; only retrieval heads read)
 *   w_q_idx bf16 [Hq_r][D][I]       query projections; head c starts at c*w_head_stride
 *                                   elements (w_head_stride == 0: one matrix shared by all)
 *   k_idx   bf16 [B][Hkv_r][n_cap][I]   stored pre-RoPE key projections
 *   scores  fp32 [B][Hq_r][n_cap]   written for j < n_ctx
 *   row_max, row_sum fp32 [B][Hq_r]
 * n_ctx in [1, n_cap].  A layer with no retrieval head is valid and does nothing.
 */
rtp_status rtp_indexer_score(const rtp_layer_desc* desc, int64_t n_ctx,
                             const uint16_t* q_pre, const uint16_t* w_q_idx, int64_t w_head_stride,
                             const uint16_t* k_idx, float idx_scale,
                             float* scores, float* row_max, float* row_sum,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_topp_select -- the query-adaptive top-p token set of every score row.
 * (abstract, observation (3): dynamic top-p instead of fixed top-k; summary,
 * "Approach": query-adaptive top-p threshold)
 *
 * With pi_j = exp(s_j - row_max) / row_sum, tokens are ranked by score (higher
 * first; equal scores: lower index first) and the set is the shortest prefix of
 * that ranking whose mass reaches top_p.  top_p >= 1 keeps all n_ctx tokens.
 * The mass is accumulated in u64 fixed point: the row max weighs 2^F with F = 42 up
 * to 2^20 tokens and one bit less per doubling beyond (the row total stays below
 * 2^63).  Sums are exact and order independent, so results are bit-reproducible; a
 * token whose rank sits within n_ctx * 2^-(F+1) of the p boundary (~1e-7 at 1M tokens)
 * may differ from an exact computation.  top_p < 1 with n_ctx > 2^24 returns
 * RTP_EUNSUPPORTED (the bound would pass 1e-4 of the mass).
 *
 *   scores   fp32 [B][Hq_r][n_cap]  (j < n_ctx read), row_max/row_sum fp32 [B][Hq_r]
 *            (row_sum is accepted for interface symmetry; the fixed-point total is used)
 *   top_p    in (0, 1]; values > 1 act as 1; <= 0 or NaN -> RTP_EINVAL
 *   sel_idx  int32 [B][Hq_r][n_cap]: the first sel_count entries of each row hold
 *            the selected token indices in increasing order; the rest is untouched
 *   sel_count int32 [B][Hq_r]
 *   sel_starts int32 [B][Hq_r][ceil(n_ctx / RTP_SEL_RANGE) + 1] or NULL: a range
 *            index of each selected list, entry q = number of selected tokens with
 *            index < q * RTP_SEL_RANGE (the last entry = sel_count).  Optional; when
 *            given, rtp_sparse_decode_attn can take it instead of rebuilding it.
 * The row_max values are the reference of every weight exp(s - row_max): pass the
 * row maxima rtp_indexer_score wrote (a smaller value saturates weights at 1).
 * The workspace holds the radix histograms, row states, counters, per-range
 * records and per-range digit tables of the search (rtp_workspace_bytes grows by
 * 2 bytes per token of n_cap per row for the tables); see the zero-fill rule above.
 */
rtp_status rtp_topp_select(const rtp_layer_desc* desc, int64_t n_ctx,
                           const float* scores, const float* row_max, const float* row_sum,
                           float top_p, int32_t* sel_idx, int32_t* sel_count, int32_t* sel_starts,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_topk_select -- the static fixed-budget rule the abstract contrasts with
 * top-p (abstract, observation (3); summary, "Key results": top-k baseline): the
 * k tokens that rank first by (score descending, index ascending).
 *
 *   scores   fp32 [B][Hq_r][n_cap] (j < n_ctx read)
 *   k        >= 1; k >= n_ctx keeps all n_ctx tokens
 *   sel_idx, sel_count, sel_starts   as rtp_topp_select (sel_count = min(k, n_ctx))
 * Same radix search as rtp_topp_select with every token weighing 1, so the
 * result is exact (integer work) and bit-reproducible.  Workspace: the
 * RTP_CALL_TOPP_SELECT size, under the same zero-fill rule.
 */
rtp_status rtp_topk_select(const rtp_layer_desc* desc, int64_t n_ctx, const float* scores, int64_t k,
                           int32_t* sel_idx, int32_t* sel_count, int32_t* sel_starts,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_sparse_decode_attn -- decode attention of the retrieval heads over their
 * selected tokens only (abstract: sparse attention through the token indexer).
 *
 *   out[b,h] = sum_{j in S(b,c)} softmax_j(sm_scale * q[b,h].k[b,g,j]) v[b,g,j]
 *
 *   q        bf16 [B][Hq][D]  post-RoPE queries
 *   k_cache, v_cache bf16 [B][Hkv][n_cap][D]
 *   sel_idx, sel_count  as written by rtp_topp_select (indices < n_ctx, increasing);
 *            an entry outside [0, n_ctx) is ignored, so no cache row at or past n_ctx
 *            is read whatever the lists hold
 *   sel_starts  the range index rtp_topp_select wrote for the same sets, or NULL
 *            (then it is rebuilt from sel_idx in the workspace)
 *   out      bf16 [B][Hq][D]; only retrieval heads' rows are written.  A row
 *            with sel_count == 0 is written as zeros.
 * Rows of one GQA group are processed together: a cached row selected by several
 * heads of the group is read from HBM once.
 */
rtp_status rtp_sparse_decode_attn(const rtp_layer_desc* desc, int64_t n_ctx,
                                  const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* sel_idx, const int32_t* sel_count, const int32_t* sel_starts,
                                  float sm_scale, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_window_sink_attn -- decode attention of the local heads over
 * [0, min(n_sinks, n_ctx)) U [max(0, n_ctx - window), n_ctx): sinks plus a sliding
 * window that includes the query token (summary, "Approach").
 *
 *   q bf16 [B][Hq][D]; k_cache, v_cache bf16 [B][Hkv][n_cap][D];
 *   out bf16 [B][Hq][D]: only local heads' rows are written.
 * The two decode calls write disjoint rows of `out`, so they may run concurrently
 * on different streams (with distinct workspaces).
 */
rtp_status rtp_window_sink_attn(const rtp_layer_desc* desc, int64_t n_ctx,
                                const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                float sm_scale, uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_prefill_attn -- one causal prefill chunk of one sequence (batch must be 1):
 * query rows at absolute positions [c0, c0 + C).
 *   - retrieval heads: dense causal attention, row i over keys [0, i]
 *     (summary, "Limitations": retrieval heads stay dense in prefill);
 *   - local heads: row i over [0, min(n_sinks, i+1)) U [max(0, i-window+1), i]
 *     (summary, "Approach");
 *   - the chunk's indexer keys, k_idx_cache[r][c0+t] = bf16(k_pre[t][g(r)] . W_k_idx[r]),
 *     for every retrieval KV head (pre-RoPE key projection, summary "Approach").
 *
 *   q        bf16 [C][Hq][D]  post-RoPE queries of the chunk
 *   k_cache, v_cache bf16 [Hkv][n_cap][D]: rows [0, c0 + C) valid (the caller has
 *            appended the chunk's post-RoPE keys and values)
 *   k_pre    bf16 [C][Hkv][D] pre-RoPE keys of the chunk (retrieval heads read)
 *   w_k_idx  bf16 [Hkv_r][D][I]; head r starts at r*w_head_stride (0 = shared)
 *   k_idx_cache bf16 [Hkv_r][n_cap][I]: rows [c0, c0+C) are written
 *   out      bf16 [C][Hq][D]
 * Requires c0 >= 0, C >= 1, c0 + C <= n_cap; head_dim 64 or 128 (each has its own
 * kernel instantiation: tile layout and MFMA schedule).
 */
rtp_status rtp_prefill_attn(const rtp_layer_desc* desc, int64_t c0, int32_t C,
                            const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            const uint16_t* k_pre, const uint16_t* w_k_idx, int64_t w_head_stride,
                            uint16_t* k_idx_cache, float sm_scale, uint16_t* out,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_decode_step -- one whole decode step of a layer in one call: exactly
 *   rtp_indexer_score -> rtp_topp_select -> rtp_sparse_decode_attn, and
 *   rtp_window_sink_attn, with the same arguments and the same results bit for
 *   bit (abstract, observations (1)-(3); summary, "Approach").
 * It enqueues seven launches instead of thirteen: the local heads' attention
 * runs in the same launch as the indexer scoring, the first radix pass also
 * reduces the row statistics, and one merge launch serves both head kinds
 * (above 128K tokens the retrieval rows' merge takes one more launch: it
 * combines 32 split partials at a time first).
 *
 *   q_pre, w_q_idx, w_head_stride, k_idx, idx_scale   as rtp_indexer_score
 *   q, k_cache, v_cache, sm_scale                     as the decode calls (RTP_KV_COMPACT:
 *                                                     k_cache/v_cache = the retrieval cache)
 *   k_loc, v_loc   RTP_KV_COMPACT: the local heads' ring; ignored (may be NULL)
 *                  with RTP_KV_FULL
 *   top_p                                             as rtp_topp_select
 *   scores, row_max, row_sum, sel_idx, sel_count      outputs, as the separate calls
 *   sel_starts   optional output (NULL: kept in the workspace)
 *   out          bf16 [B][Hq][D]: every head's row is written
 * Pointers of the retrieval-head path may be NULL when the layer has no
 * retrieval head.  Workspace: rtp_workspace_bytes(desc, n_ctx,
 * RTP_CALL_DECODE_STEP), zero-filled before the first call (see the
 * conventions above); its selection region sits first and depends only on the
 * descriptor, so the same workspace serves every n_ctx <= n_cap of the layer.
 */
rtp_status rtp_decode_step(const rtp_layer_desc* desc, int64_t n_ctx,
                           const uint16_t* q_pre, const uint16_t* w_q_idx, int64_t w_head_stride,
                           const uint16_t* k_idx, float idx_scale,
                           const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                           const uint16_t* k_loc, const uint16_t* v_loc,
                           float top_p, float sm_scale,
                           float* scores, float* row_max, float* row_sum,
                           int32_t* sel_idx, int32_t* sel_count, int32_t* sel_starts,
                           uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * Growing-context generation with the context length on the device, so that one
 * captured HIP graph of [rtp_append_token_dev, rtp_decode_step_dev] serves every new
 * token (a long generation grows the retrieval heads' context by one token per step;
 * abstract: full KV kept for retrieval heads; summary, "Experimental setup": long
 * reasoning outputs).
 *
 * gen: int64_t[2] in DEVICE memory, {pos, n_ctx}, 8-byte aligned, caller-owned:
 *   rtp_append_token_dev stores the token at position gen[0] exactly as
 *   rtp_append_token(pos = gen[0]) does and sets gen[1] = gen[0] + 1 (clamped to
 *   [1, n_cap]; a position outside [0, n_cap) writes nothing);
 *   rtp_decode_step_dev computes exactly what rtp_decode_step computes for
 *   n_ctx = gen[1] (clamped to [1, n_max]) and, in its last launch, sets
 *   gen[0] = gen[1].
 * A replay of the pair therefore appends the next token and decodes over it.  The
 * caller writes the new token's k/v/k_pre into the same buffers before each replay.
 *
 * rtp_decode_step_dev: n_max is the longest context the call will see (the grids,
 * strides and workspace are sized for it: rtp_workspace_bytes(desc, n_max,
 * RTP_CALL_DECODE_STEP)); the other arguments are rtp_decode_step's.  sel_starts rows
 * are n_max's (row stride ceil(n_max / RTP_SEL_RANGE) + 1; entry ceil(n_ctx /
 * RTP_SEL_RANGE) holds the count).  Where the layout of the split partials differs
 * between n_max and n_ctx (window lists shorter than the window, or selection tiles of
 * another size), the outputs can differ from rtp_decode_step's in rounding only.
 */
rtp_status rtp_append_token_dev(const rtp_layer_desc* desc, int64_t* gen,
                                const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_pre,
                                const uint16_t* w_k_idx, int64_t w_head_stride,
                                uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache,
                                uint16_t* k_loc, uint16_t* v_loc, void* stream);
rtp_status rtp_decode_step_dev(const rtp_layer_desc* desc, int64_t n_max, int64_t* gen,
                               const uint16_t* q_pre, const uint16_t* w_q_idx, int64_t w_head_stride,
                               const uint16_t* k_idx, float idx_scale,
                               const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                               const uint16_t* k_loc, const uint16_t* v_loc,
                               float top_p, float sm_scale,
                               float* scores, float* row_max, float* row_sum,
                               int32_t* sel_idx, int32_t* sel_count, int32_t* sel_starts,
                               uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * rtp_decode_step_noalloc -- rtp_decode_step for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same launches, arguments and results bit for bit, with the workspace
 * replaced by a scratch array the library holds on each GPU it runs on
 * (rtp_decode_step_noalloc_max_bytes() bytes, 64 MiB, kept until the process ends).
 * It calls no allocating routine: the array's device address is looked up on the first
 * call on a device, and every call zero-fills the part the step needs zero with a kernel
 * (no memset node).
 *   - A layer and context whose workspace (rtp_workspace_bytes(desc, n_ctx,
 *     RTP_CALL_DECODE_STEP)) exceeds the array returns RTP_EUNSUPPORTED, nothing enqueued.
 *   - All calls on one GPU share its array: calls whose execution overlaps (other
 *     streams, other threads, other graphs replaying) race and give wrong results; the
 *     caller serialises them.
 */
size_t rtp_decode_step_noalloc_max_bytes(void);
rtp_status rtp_decode_step_noalloc(const rtp_layer_desc* desc, int64_t n_ctx,
                                   const uint16_t* q_pre, const uint16_t* w_q_idx, int64_t w_head_stride,
                                   const uint16_t* k_idx, float idx_scale,
                                   const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                   const uint16_t* k_loc, const uint16_t* v_loc,
                                   float top_p, float sm_scale,
                                   float* scores, float* row_max, float* row_sum,
                                   int32_t* sel_idx, int32_t* sel_count, int32_t* sel_starts,
                                   uint16_t* out, void* stream);

/*
 * rtp_append_token -- store the token at position `pos` (the next one; decode then
 * runs with n_ctx = pos + 1) in every cache of the layout: its post-RoPE key and
 * value for every head, and for retrieval heads its indexer key
 * k_idx_cache[b][r][pos] = bf16(k_pre[b][g(r)] . W_k_idx[r]) (fp32 accumulation,
 * one rounding; abstract, observation (2); summary, "Approach").
 *
 *   k_new, v_new  bf16 [B][Hkv][D] post-RoPE;  k_pre bf16 [B][Hkv][D] pre-RoPE
 *   w_k_idx       bf16 [Hkv_r][D][I], head r at r*w_head_stride (0 = shared)
 *   RTP_KV_FULL:    k_cache/v_cache [B][Hkv][n_cap][D]; k_loc/v_loc ignored
 *   RTP_KV_COMPACT: k_cache/v_cache [B][Hkv_r][n_cap][D] (retrieval heads) and
 *                   k_loc/v_loc [B][Hkv_l][n_sinks + window][D] (the ring)
 *   k_idx_cache   bf16 [B][Hkv_r][n_cap][I]
 * Requires 0 <= pos < n_cap.  Pointers of a head kind the layer lacks may be NULL.
 */
rtp_status rtp_append_token(const rtp_layer_desc* desc, int64_t pos,
                            const uint16_t* k_new, const uint16_t* v_new, const uint16_t* k_pre,
                            const uint16_t* w_k_idx, int64_t w_head_stride,
                            uint16_t* k_cache, uint16_t* v_cache, uint16_t* k_idx_cache,
                            uint16_t* k_loc, uint16_t* v_loc, void* stream);

/*
 * rtp_hbm_read_probe -- diagnostic: stream `bytes` of `buf` (device, 16-byte
 * aligned) through plain 16-byte loads and discard them (sink: a device word that is
 * almost never written).  Timing it gives the device's practical HBM read rate, the
 * reference against which the decode kernels' bandwidth is read; it is not part of
 * the method.
 */
rtp_status rtp_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * rtp_mfma_probe -- diagnostic: every wave of 2 blocks per compute unit (2 waves per
 * SIMD) runs `iters` trips of 4 independent v_mfma_f32_32x32x16_bf16 chains from
 * register operands (the prefill's MFMA shape); *flops (HOST) receives the launch's
 * flop count, sink is a device word that is almost never written.  Timing it gives
 * the dense bf16 MFMA rate the chip sustains (its clock under such a load), the
 * reference against which the prefill's MFMA rate is read; it is not part of the method.
 * iters in [1, 2^24].
 */
rtp_status rtp_mfma_probe(uint32_t iters, float* sink, double* flops, void* stream);

/* Human-readable name of a status code (static string). */
const char* rtp_status_string(rtp_status s);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* rtp_last_error(void);

/* Library version string. */
const char* rtp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H */
