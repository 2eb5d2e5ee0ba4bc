/*
 * dash.h -- C ABI of the DashAttention forward path on MI355X (gfx950).
 *
 * DashAttention has three phases; each entry point below runs one or more of
 * them on the GPU.  The phases are defined in the technical summary
 * "Technische Samenvatting: DashAttention" (gist.science/nl/paper/2605.18753):
 *   phase 0  "Fase 0: Lokale Chunk Samenvatting"   learned-query chunk summaries
 *   phase 1  "Fase 1: Entmax Chunk Routering"      alpha-entmax routing, GQA
 *            averaging, equation  w_hat = alpha-entmax(gamma * z_bar)
 *   phase 2  "Fase 2: Prior-Geinduceerde Spaarzame Softmax"  prior-induced
 *            sparse softmax over the active chunks plus the diagonal branch
 * and the interface (q, k, v, a per-head summary query "head_cls", chunk_size,
 * enable_gqa, an optional active_blocks output) in the aiexpert.news article
 * "DashAttention alcanza 75% de dispersidad ...", interface paragraph.
 *
 * Conventions shared by every call
 * --------------------------------
 * Memory.   Every tensor argument is a DEVICE pointer to contiguous row-major
 *           memory owned by the caller.  The library never allocates or frees
 *           memory; scratch space comes from a caller-provided workspace of at
 *           least dash_workspace_size(op, shape) bytes (256-byte aligned).
 *           q/k/v/out/summaries must be 16-byte aligned.
 * Layout.   Token-major packed "THD": q [T, Hq, D], k and v [T, Hkv, D].
 *           Sequence s occupies rows cu_seqlens[s] .. cu_seqlens[s+1]-1, or
 *           rows s*max_seqlen .. (s+1)*max_seqlen-1 when cu_seqlens is NULL.
 *           Chunk c of a sequence holds its tokens c*B .. c*B+B-1; only
 *           complete chunks have a summary.  Summaries of all sequences are
 *           packed in sequence order: k_bar [sum_s floor(L_s/B), Hkv, D].
 * Heads.    With enable_gqa = 0, Hq must equal Hkv.  With enable_gqa = 1,
 *           Hq must be a multiple of Hkv; query head q reads KV head
 *           floor(q / (Hq/Hkv)) (the repeat-interleave convention).
 * Routing.  A query at local position i routes to the chunks c < floor(i/B)
 *           of its own sequence; its own chunk is the diagonal branch,
 *           attended causally with bias 0.  The mask row of (KV head h,
 *           token t) is W = ceil(C_slots/64) 64-bit words, chunk c in bit
 *           (c % 64) of word c / 64 (least significant bit first), with
 *           C_slots = ceil(max_seqlen / B).  Bits c >= floor(i/B) are zero.
 * Streams.  Every call only enqueues work on `stream` (a hipStream_t; NULL is
 *           the default stream) and never synchronises.
 * Errors.   All host-visible arguments are checked before any HIP call; on
 *           an error nothing is enqueued and nothing is written.  A failed
 *           kernel launch returns DASH_ERR_HIP.  Device-side contents
 *           (cu_seqlens, seqlens, alpha_per_seq) are preconditions and are
 *           not checked.  The only global state is the per-device scratch
 *           of dash_attn_decode_noalloc (its address, looked up once per
 *           device under a lock); every other entry point uses only its
 *           arguments, so calls from several host threads are safe; calls
 *           that share output or workspace buffers must be ordered by the
 *           caller.
 * Supported: head_dim in {64, 128}; chunk_size in {64, 128}; dtype bf16 or
 *           fp32 (q, k, v, summaries and out share it; accumulation is fp32);
 *           C_slots <= 2048; alpha in [1, 2].  In bf16 the GQA group size
 *           Hq/Hkv must be 1, 2, 4, 8, 16 or 32.  Anything else returns
 *           DASH_ERR_UNSUPPORTED.
 */
#ifndef DASH_H_
#define DASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DASH_ABI_VERSION 3

typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARGUMENT = 1,
  DASH_ERR_UNSUPPORTED = 2,
  DASH_ERR_WORKSPACE_TOO_SMALL = 3,
  DASH_ERR_HIP = 4
} dash_status;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype;

typedef enum {
  DASH_OP_SUMMARIZE = 0,
  DASH_OP_ROUTE = 1,
  DASH_OP_PREFILL = 2,
  DASH_OP_DECODE = 3,
  DASH_OP_SPARSE = 4,
  DASH_OP_DECODE_SPARSE = 5,
  DASH_OP_ROUTE_DECODE = 6,    /* dash_route_topk on decode rows */
  DASH_OP_BACKWARD = 7,        /* dash_attn_sparse_backward */
  DASH_OP_PREFILL_BACKWARD = 8 /* dash_attn_prefill_backward */
} dash_op;

typedef struct {
  int32_t num_seqs;            /* sequences (prefill) or batch entries (decode)   */
  int32_t max_seqlen;          /* fixed length, or an upper bound on every length;
                                  decode: cache capacity per sequence             */
  int64_t total_tokens;        /* T, rows of q/k/v; must be num_seqs*max_seqlen
                                  when cu_seqlens is NULL; ignored by decode      */
  const int32_t* cu_seqlens;   /* device [num_seqs+1] prefix sums, or NULL        */
  int32_t num_q_heads;         /* Hq  */
  int32_t num_kv_heads;        /* Hkv */
  int32_t head_dim;            /* D   */
  int32_t chunk_size;          /* B   */
  int32_t dtype;               /* dash_dtype of q, k, v, summaries and out        */
} dash_shape;

/* Derived sizes of a shape, for sizing caller buffers.  Returns DASH_OK or
 * the status the shape itself would produce. */
typedef struct {
  int64_t summary_rows;        /* rows of k_bar the caller must provide: floor(T/B)
                                  (prefill), num_seqs*max_seqlen/B (decode cache) */
  int32_t chunk_slots;         /* C_slots = ceil(max_seqlen / B)                  */
  int32_t mask_words;          /* W = ceil(C_slots / 64)                          */
  int32_t group_size;          /* G = Hq / Hkv                                    */
} dash_layout;

dash_status dash_get_layout(const dash_shape* shape, int enable_gqa, dash_layout* out);

/* Phase 0 ("Fase 0: Lokale Chunk Samenvatting").  For every KV head h and
 * complete chunk c of every sequence, a learned query q_bar[h] attends to the
 * chunk's keys with local scaled dot-product attention (scale 1/sqrt(D)), the
 * keys serving as values:
 *     k_bar[c,h] = sum_t softmax_t(<q_bar[h], k[cB+t,h]> / sqrt(D)) k[cB+t,h].
 * q_bar = 0 gives the mean of the chunk's keys.  Accumulation is fp32; a bf16
 * result is rounded to nearest even once.
 *   k     [T, Hkv, D] dtype                  (input)
 *   qbar  [Hkv, D] fp32                      (input)
 *   kbar  [>= summary_rows, Hkv, D] dtype    (output; rows past the last
 *                                             complete chunk are not written)
 * For a decode cache pass the cache as a fixed-length batch
 * (cu_seqlens = NULL, max_seqlen = capacity, total_tokens = batch*capacity);
 * the result is then k_bar [batch, capacity/B, Hkv, D]. */
dash_status dash_summarize(const dash_shape* shape, const void* k, const float* qbar,
                           void* kbar, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Estimated summary of each position's own, partial chunk, for the
 * estimate_diagonal option.  The interface carries estimate_diagonal as a
 * diagonal correction of the alpha-entmax normalisation (aiexpert.news
 * article, the interface paragraph); the pages define it no further.  The
 * reading taken: position i's chunk c = floor(i/B) has no summary yet, so it
 * gets phase 0's attention over the keys it has so far,
 *     k_diag[t,h] = sum_{j=cB..i} softmax_j(<q_bar[h], k[j,h]> / sqrt(D)) k[j,h],
 * which equals k[t,h] at i = cB and the chunk's summary at i = cB + B - 1.
 * Passed to dash_route it enters every head's entmax as one more entry.
 *   k      [T, Hkv, D] dtype                 (input)
 *   qbar   [Hkv, D] fp32                     (input)
 *   kdiag  [T, Hkv, D] dtype                 (output) */
dash_status dash_summarize_diagonal(const dash_shape* shape, const void* k, const float* qbar,
                                    void* kdiag, void* stream);

/* Phase 1 ("Fase 1: Entmax Chunk Routering").  For token t at local position
 * i and query head q (KV head h):
 *     u_c     = gamma * s * <q[t,q], k_bar[c,h]>            c < floor(i/B)
 *     p       = alpha-entmax(u):  p_c = [(alpha-1) u_c - tau]_+^(1/(alpha-1)),
 *               sum_c p_c = 1 (alpha = 1: softmax; every chunk active)
 *     w_bar_c = mean over the G query heads of KV head h of p_c
 *     bit_c   = OR over those heads of [u_c > tau_hat],  tau_hat = tau/(alpha-1)
 *     log_prior_c = sigma * log(w_bar_c) where bit_c = 1
 * s = softmax_scale, or 1/sqrt(D) when softmax_scale <= 0.  With kdiag, a row
 * with routable chunks also has the entry u_d = gamma * s * <q[t,q],
 * kdiag[t,h]> in each head's entmax (after the routed chunks); it takes its
 * share of the unit mass and enters tau, but never a mask bit or a prior.
 *   q              [T, Hq, D] dtype                (input)
 *   kbar           [summary_rows, Hkv, D] dtype    (input)
 *   kdiag          [T, Hkv, D] dtype or NULL       (input, dash_summarize_diagonal)
 *   alpha          used when alpha_per_seq is NULL; 1 <= alpha <= 2
 *   alpha_per_seq  device fp32 [num_seqs] or NULL
 *   active_blocks  [Hkv, T, W] uint64              (output, required)
 *   log_prior      [Hkv, T, C_slots] fp32 or NULL  (output; slots c < floor(i/B)
 *                                                   are written, -inf where the
 *                                                   bit is 0)
 *   tau            [Hq, T] fp32 or NULL            (output: tau_hat in u units;
 *                                                   +inf when no chunk is
 *                                                   routable, -inf for alpha=1) */
dash_status dash_route(const dash_shape* shape, const void* q, const void* kbar,
                       const void* kdiag, float alpha, const float* alpha_per_seq,
                       float gamma, float sigma, float softmax_scale, int enable_gqa,
                       uint64_t* active_blocks, float* log_prior, float* tau,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Phases 0-2, causal prefill ("Fase 2: Prior-Geinduceerde Spaarzame Softmax").
 * Runs dash_summarize and dash_route into the workspace, then for every token
 * t at position i and query head q:
 *     o[t,q] = sum_j softmax_j(s <q[t,q], k[j,h]> + b_j) v[j,h]
 * over the keys j of the active routed chunks (b_j = log_prior of j's chunk)
 * and the causal diagonal chunk floor(i/B)*B <= j <= i (b_j = 0).
 *   q, k, v        [T, Hq|Hkv, D] dtype            (input)
 *   qbar           [Hkv, D] fp32                   (input)
 *   estimate_diagonal  nonzero: route with dash_summarize_diagonal's estimates
 *   out            [T, Hq, D] dtype                (output)
 *   lse            [Hq, T] fp32 or NULL            (output, natural log of the
 *                                                   softmax denominator)
 *   active_blocks  [Hkv, T, W] uint64 or NULL      (output) */
dash_status dash_attn_prefill(const dash_shape* shape, const void* q, const void* k,
                              const void* v, const float* qbar, float alpha,
                              const float* alpha_per_seq, float gamma, float sigma,
                              float softmax_scale, int enable_gqa, int estimate_diagonal,
                              void* out, float* lse, uint64_t* active_blocks, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Phase 2 alone ("Fase 2: Prior-Geinduceerde Spaarzame Softmax", the
 * FlashAttention-style kernel that walks a bit-packed mask and adds the
 * routing bias before the softmax): the attention step of dash_attn_prefill
 * for a given routing.  dash_attn_prefill is exactly dash_summarize, then
 * dash_route, then this call.
 *   q, k, v        [T, Hq|Hkv, D] dtype            (input)
 *   active_blocks  [Hkv, T, W] uint64              (input, as dash_route writes it;
 *                                                   bits c >= floor(i/B) must be 0)
 *   log_prior      [Hkv, T, C_slots] fp32          (input; read where a bit is set)
 *   out            [T, Hq, D] dtype                (output)
 *   lse            [Hq, T] fp32 or NULL            (output)
 * The workspace (dash_workspace_size(DASH_OP_SPARSE, ...)) holds a transposed
 * copy of V for bf16 inputs with a GQA group of 16 or more. */
dash_status dash_attn_sparse(const dash_shape* shape, const void* q, const void* k,
                             const void* v, const uint64_t* active_blocks,
                             const float* log_prior, float softmax_scale, int enable_gqa,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             void* stream);

/* One incremental decode step: each batch entry b has one new query whose
 * key and value are already written at position seqlens[b]-1 of its cache.
 * Routes that query against the cached summaries of its complete chunks
 * (summaries are fixed and cached once a chunk is complete, "Fase 0",
 * Efficientie bullet) and attends as dash_attn_prefill does for its last row.
 * shape: num_seqs = batch, max_seqlen = cache capacity (a multiple of B),
 * cu_seqlens = NULL.
 *   q              [batch, Hq, D] dtype            (input)
 *   k_cache,v_cache[batch, capacity, Hkv, D] dtype (input)
 *   seqlens        device int32 [batch], 1 <= seqlens[b] <= capacity
 *   kbar_cache     [batch, capacity/B, Hkv, D] dtype (input; rows c <
 *                                                   floor((seqlens[b]-1)/B) read)
 *   qbar           [Hkv, D] fp32 (input; read only with estimate_diagonal)
 *   estimate_diagonal  nonzero: the new row's own-chunk estimate (keys
 *                  floor((L-1)/B)*B .. L-1 of its cache, as
 *                  dash_summarize_diagonal) joins its routing
 *   out            [batch, Hq, D] dtype            (output)
 *   lse            [Hq, batch] fp32 or NULL        (output)
 *   active_blocks  [Hkv, batch, W] uint64 or NULL  (output) */
dash_status dash_attn_decode(const dash_shape* shape, const void* q,
                             const void* k_cache, const void* v_cache,
                             const int32_t* seqlens, const void* kbar_cache,
                             const float* qbar, float alpha, float gamma, float sigma,
                             float softmax_scale, int enable_gqa, int estimate_diagonal,
                             void* out, float* lse, uint64_t* active_blocks, void* workspace,
                             size_t workspace_bytes, void* stream);

/* dash_cache_append and dash_attn_decode as one fused step: the new tokens'
 * K/V rows go to position seqlens[b]-1 of the caches, the chunk each of them
 * completes is summarised into kbar_cache, and the new queries are decoded
 * over the updated caches.  A chunk's summary is computed once, by the step
 * whose token completes it, "fused into the decode step" (incremental
 * decoding: "Belangrijkste Bijdragen", the GPU implementation item, of the
 * gist.science summary; "Fase 0", Efficientie bullet, for the cached
 * summaries).  For bf16 without estimate_diagonal the append runs inside the
 * routing's first launch, beside the logits (which never read what it
 * writes: a query routes only the chunks before its own); otherwise it is a
 * launch of its own before the step.  Results equal dash_cache_append then
 * dash_attn_decode with the same arguments, bit for bit.
 * Arguments as dash_attn_decode and dash_cache_append, with:
 *   k_new, v_new   [batch, Hkv, D] dtype            (input)
 *   k_cache,v_cache[batch, capacity, Hkv, D] dtype  (in/out: row L-1 written)
 *   kbar_cache     [batch, capacity/B, Hkv, D] dtype (in/out: row L/B-1 written
 *                                                    when L % B == 0)
 *   qbar           [Hkv, D] fp32                    (input, required)
 *   workspace      dash_workspace_size(DASH_OP_DECODE, shape) bytes
 * NULL or misaligned k_new / v_new / qbar: DASH_ERR_INVALID_ARGUMENT. */
dash_status dash_attn_decode_append(const dash_shape* shape, const void* q, const void* k_new,
                                    const void* v_new, void* k_cache, void* v_cache,
                                    const int32_t* seqlens, void* kbar_cache, const float* qbar,
                                    float alpha, float gamma, float sigma, float softmax_scale,
                                    int enable_gqa, int estimate_diagonal, void* out, float* lse,
                                    uint64_t* active_blocks, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* dash_attn_decode for callers that cannot allocate device memory: code that
 * runs under HIP graph capture, tight serving loops, and hosts that forbid
 * allocation.  Same arguments, layout and results as dash_attn_decode, without
 * the workspace: its intermediates (routing logits and thresholds, mask and
 * log-prior, split-K partials) live in a scratch array of
 * DASH_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * copy per GPU, for the life of the process.  Nothing is allocated or freed
 * by this call.
 *   Limit: a shape whose decode workspace (dash_noalloc_scratch_need) exceeds
 *          DASH_NOALLOC_SCRATCH_BYTES returns DASH_ERR_UNSUPPORTED; use
 *          dash_attn_decode with a workspace of its size instead.
 *   The stream's device must be the current device (else
 *          DASH_ERR_INVALID_ARGUMENT); the first call on a device looks up the
 *          scratch's address there (under a lock), later calls reuse it.
 *   Every call on one GPU shares that GPU's scratch and leaves its last
 *          contents there: calls that overlap in time on one GPU (on
 *          different streams, or from several host threads without ordering)
 *          race and give undefined results.  Calls on one stream are ordered
 *          and safe.  No part of the scratch needs to start at zero. */
#define DASH_NOALLOC_SCRATCH_BYTES (32u << 20)
dash_status dash_attn_decode_noalloc(const dash_shape* shape, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* seqlens, const void* kbar_cache,
                                     const float* qbar, float alpha, float gamma, float sigma,
                                     float softmax_scale, int enable_gqa,
                                     int estimate_diagonal, void* out, float* lse,
                                     uint64_t* active_blocks, void* stream);
/* Scratch bytes dash_attn_decode_noalloc needs for a decode shape (0 if the
 * shape is invalid or unsupported). */
size_t dash_noalloc_scratch_need(const dash_shape* shape);

/* The work list the G >= 16 bf16 prefill attention runs a packed (varlen)
 * batch by (exposed for inspection): one entry per (sequence, tile of P
 * consecutive positions), (sequence << 16) | tile, cost-sorted -- the
 * sequences longest first (by tile count, ties by index), each sequence's
 * tiles from its last (a tile's rows see more keys the later it starts) down
 * to its first -- then 0xffffffff up to `capacity`.  The grid is sized by
 * this list, not by num_seqs x max_seqlen.  The scheduling side of "iterate
 * over the active chunks" ("Fase 2", the implementation bullet of the
 * gist.science summary) for sequences of mixed lengths.
 *   shape          varlen prefill shape (cu_seqlens set), bf16, G in {16, 32},
 *                  num_seqs <= 1024 (else DASH_ERR_UNSUPPORTED)
 *   items          device uint32 [capacity]          (output)
 *   capacity       >= ceil(T / 8) + num_seqs (else DASH_ERR_WORKSPACE_TOO_SMALL)
 *   positions_per_tile  host int                     (output: P) */
dash_status dash_prefill_schedule(const dash_shape* shape, int enable_gqa, uint32_t* items,
                                  size_t capacity, int* positions_per_tile, void* stream);

/* Measurement probe (not part of the attention path): one launch that
 * measures an achievable peak of this GPU, to read the kernels' roofline
 * fractions against next to the published peaks.
 *   kind 0: MFMA issue loop, two independent 16x16x32 bf16 accumulator
 *           chains per wave, two waves per SIMD, `iters` rounds (src unused);
 *   kind 1: HBM read stream of `bytes` (a multiple of 16) from src with
 *           16-byte loads (iters unused).
 *   sink   >= 1024 bytes of device memory (written only on a bit pattern the
 *          probes never produce)
 *   work   host double: FLOPs (kind 0) or bytes (kind 1) the launch processes
 * Time the launch with events on `stream`. */
dash_status dash_probe_peak(int kind, const void* src, size_t bytes, int iters, void* sink,
                           size_t sink_bytes, double* work, void* stream);

/* Decode-cache upkeep for incremental decoding: appends one new token per
 * batch entry to the K/V caches and keeps the summary cache current.  A
 * chunk's summary is fixed once the chunk is complete, so it is computed once,
 * by the append that completes it, and cached ("Fase 0", Efficientie bullet;
 * incremental decoding: "Belangrijkste Bijdragen", the GPU implementation
 * item, of the same page).  With L = seqlens[b]
 * (the length after the append, 1 <= L <= capacity), the token's key and
 * value go to position L-1; when L % B == 0 the summary of chunk L/B - 1 is
 * computed from the chunk's B keys (as dash_summarize does) and written to
 * kbar_cache.  Call it before dash_attn_decode with the same seqlens.
 * shape as in dash_attn_decode.
 *   k_new, v_new   [batch, Hkv, D] dtype           (input)
 *   seqlens        device int32 [batch]            (input; entries are not checked)
 *   qbar           [Hkv, D] fp32                   (input)
 *   k_cache,v_cache[batch, capacity, Hkv, D] dtype (in/out: row L-1 written)
 *   kbar_cache     [batch, capacity/B, Hkv, D] dtype (in/out: row L/B-1 written when
 *                                                   L % B == 0)
 * No workspace.  Calls on one stream see each other's writes in order. */
dash_status dash_cache_append(const dash_shape* shape, const void* k_new, const void* v_new,
                              const int32_t* seqlens, const float* qbar, void* k_cache,
                              void* v_cache, void* kbar_cache, void* stream);

/* Top-k block routing, the comparison mode of the hierarchical methods the
 * pages set DashAttention against: NSA and InfLLMv2 keep a fixed number of
 * KV blocks ranked by a coarse score and then run ordinary softmax attention
 * over the kept tokens ("Technische Samenvatting: DashAttention",
 * Probleemstelling; the same point in the Paper Overview and in the
 * aiexpert.news article).  The pages do not define
 * the coarse score; here it is the group-shared score
 *     S_c = sum over the G query heads of KV head h of softmax_c(u_c),
 *     u_c = gamma * s * <q[t,q], k_bar[c,h]>        c < floor(i/B),
 * the routing logits of dash_route.  The min(topk, floor(i/B)) chunks of
 * largest S_c are active (equal scores: lower chunk index first) and the
 * log-prior is 0 on them (-inf elsewhere), so dash_attn_sparse /
 * dash_attn_decode_sparse then run plain softmax attention over the selected
 * chunks and the diagonal.  (Dense causal attention on the same kernels is
 * dash_route with alpha = 1, sigma = 0: every routable chunk, bias 0.)
 *   topk           >= 1
 *   decode_seqlens NULL: prefill rows, as dash_route (q [T, Hq, D], kbar
 *                  [summary_rows, Hkv, D], workspace DASH_OP_ROUTE);
 *                  device int32 [batch]: one decode row per batch entry at
 *                  position seqlens[b]-1, shape and kbar as in
 *                  dash_attn_decode (q [batch, Hq, D]), workspace
 *                  DASH_OP_ROUTE_DECODE (logits and scores of the rows).
 *   active_blocks  [Hkv, rows, W] uint64           (output, required)
 *   log_prior      [Hkv, rows, C_slots] fp32 or NULL (output) */
dash_status dash_route_topk(const dash_shape* shape, const void* q, const void* kbar,
                            int topk, float gamma, float softmax_scale, int enable_gqa,
                            const int32_t* decode_seqlens, uint64_t* active_blocks,
                            float* log_prior, void* workspace, size_t workspace_bytes,
                            void* stream);

/* The attention step of dash_attn_decode ("Fase 2", split-K over the active
 * chunks plus the diagonal, then the merge of the splits) for a given routing:
 * dash_attn_decode is its routing of the new tokens followed by this call.
 * shape as in dash_attn_decode.
 *   q, k_cache, v_cache, seqlens  as in dash_attn_decode
 *   active_blocks  [Hkv, batch, W] uint64          (input; bits c >=
 *                                                   floor((seqlens[b]-1)/B) must be 0)
 *   log_prior      [Hkv, batch, C_slots] fp32      (input; read where a bit is set)
 *   out            [batch, Hq, D] dtype            (output)
 *   lse            [Hq, batch] fp32 or NULL        (output)
 * Workspace: dash_workspace_size(DASH_OP_DECODE_SPARSE, shape). */
dash_status dash_attn_decode_sparse(const dash_shape* shape, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* seqlens, const uint64_t* active_blocks,
                                    const float* log_prior, float softmax_scale,
                                    int enable_gqa, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Backward of phase 2 for a given routing: the gradients of sum(dout * out)
 * for out = dash_attn_sparse(q, k, v, active_blocks, log_prior), with respect
 * to q, k, v and to the log-prior of every active routed chunk.  The pages
 * make the whole hierarchy differentiable (alpha-entmax instead of top-k lets
 * gradients reach the routing: "Technische Samenvatting: DashAttention",
 * Fase 1, Differentieerbaarheid bullet); for the attention step this is the
 * derivative of the softmax with an additive bias:
 *     P = softmax(s q k^T + b),  D_i = <dO_i, O_i>,  dS = P (dO v^T - D),
 *     dq = s dS k,  dk = s dS^T q,  dv = P^T dO,
 *     dbias[h,i,c] = sum over the chunk's keys and the group's heads of dS.
 * bf16 inputs, GQA group 16 or 32, fixed-length or packed (cu_seqlens)
 * sequences; anything else returns DASH_ERR_UNSUPPORTED.
 *   q, k, v, active_blocks, log_prior  as in dash_attn_sparse   (input)
 *   out            [T, Hq, D] dtype    (input: the forward output)
 *   dout           [T, Hq, D] dtype    (input)
 *   lse            [Hq, T] fp32        (input: the forward's LSE)
 *   dq             [T, Hq, D] dtype    (output)
 *   dk, dv         [T, Hkv, D] dtype   (output)
 *   dbias          [Hkv, T, C_slots] fp32 (output; 0 off the active routed chunks)
 * Workspace: dash_workspace_size(DASH_OP_BACKWARD, shape). */
dash_status dash_attn_sparse_backward(const dash_shape* shape, const void* q, const void* k,
                                      const void* v, const void* out, const void* dout,
                                      const float* lse, const uint64_t* active_blocks,
                                      const float* log_prior, float softmax_scale,
                                      int enable_gqa, void* dq, void* dk, void* dv,
                                      float* dbias, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Backward of the whole causal prefill (dash_attn_prefill): the gradients of
 * sum(dout * out) with respect to q, k, v and q_bar, through the attention,
 * the log-prior, the GQA mean, the alpha-entmax routing and the phase-0
 * summaries.  This is the differentiable path the pages build the method on
 * (alpha-entmax in place of top-k lets the attention's gradient reach the
 * routing and the summaries: "Technische Samenvatting: DashAttention", Fase 1,
 * Differentieerbaarheid bullet; Belangrijkste Bijdragen, item 1).  The routing
 * is recomputed from the inputs; the mask is piecewise constant and carries no
 * gradient of its own; bf16 rounding of the summaries passes gradients
 * unchanged.  The support: as dash_attn_sparse_backward.
 *   q, k, v, qbar, alpha, alpha_per_seq, gamma, sigma, softmax_scale,
 *   enable_gqa, estimate_diagonal
 *                  as in dash_attn_prefill (input); with estimate_diagonal the
 *                  gradient also flows through each row's own-chunk entry of
 *                  the entmax (it feeds no prior) and its running summary
 *   out, lse       the forward's output and LSE (input)
 *   dout           [T, Hq, D] dtype    (input)
 *   dq             [T, Hq, D] dtype    (output)
 *   dk, dv         [T, Hkv, D] dtype   (output)
 *   dqbar          [Hkv, D] fp32       (output)
 * Workspace: dash_workspace_size(DASH_OP_PREFILL_BACKWARD, shape). */
dash_status dash_attn_prefill_backward(const dash_shape* shape, const void* q, const void* k,
                                       const void* v, const float* qbar, float alpha,
                                       const float* alpha_per_seq, float gamma, float sigma,
                                       float softmax_scale, int enable_gqa,
                                       int estimate_diagonal, const void* out, const void* dout,
                                       const float* lse, void* dq, void* dk, void* dv,
                                       float* dqbar, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Workspace bytes that `op` needs for `shape` (0 when none); the same
 * enable_gqa / optional-output choices do not change it. */
size_t dash_workspace_size(int op, const dash_shape* shape);

/* Static description of a status code; never NULL. */
const char* dash_status_string(dash_status status);

/* DASH_ABI_VERSION of the built library. */
int dash_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H_ */
