/*
 * blockrank.h -- C ABI of the MI355X (gfx950) BlockRank hot path.
 *
 * BlockRank ("Scalable In-context Ranking with Generative Models") ranks N candidate
 * documents with one LLM prompt P = I || d_1 || ... || d_N || q (instruction prefix,
 * documents, final query; BlockRank blog, candidate arrangement).  This library computes,
 * for one attention layer:
 *
 *   br_attn_fwd     block-sparse prefill attention softmax(Q K^T * scale + M) V, where the
 *                   mask M lets instruction tokens read the instruction causally, each
 *                   document read the whole instruction plus itself causally, and the
 *                   final query read everything before it plus itself causally
 *                   (BlockRank summary, section 3.4 "Blockwise Structured Attention";
 *                   blog, directed-attention section: block mask with causal diagonal
 *                   blocks C).  Forbidden blocks are never computed.
 *   br_doc_scores   the attention-mass readout: for each signal query row i and head h,
 *                   a softmax of z = Q_S[i,h] . K[j, h/G] * scale over the prompt's
 *                   document tokens only, summed per document and over signal rows and
 *                   averaged over heads (BlockRank summary, "Score computation procedure"
 *                   steps 1-4; blog, attention supervision: s_k, sum_k s_k = |S|).
 *   br_sort_docs    per prompt, document indices by descending s_k (ties: lower index)
 *                   (BlockRank summary, "Efficient Attention-Based Inference" step 3;
 *                   blog, direct output).
 * and around that path:
 *   br_query_attn_fwd   query rows only, over a cached corpus (BlockSearch, section 3.2);
 *   br_attn_routed_fwd  attention over a top-B subset of the documents (BlockSearch, 5.1);
 *   br_ssmax_softmax_scale  the SSMax logit factor s ln N / sqrt(d) (BlockSearch, 5.1);
 *   br_rope_fwd, br_rope_signal_fwd  RoPE at permutation-invariant positions (BlockRank
 *                   summary, 3.4; BlockSearch, 3.2);
 *   br_attn_bwd, br_infonce, br_doc_scores_bwd  the backward of the attention, the InfoNCE
 *                   auxiliary loss and the readout (BlockRank summary, 3.4).
 *
 * Conventions (all entry points):
 *   - Every function returns br_status; BR_OK == 0.  Nothing aborts or throws.
 *   - All argument checks run on the host before any HIP call; on failure nothing is
 *     enqueued and br_last_error() (thread-local) holds a message.  A HIP runtime error
 *     maps to BR_ERR_HIP with hipGetErrorString's text.  Outputs are undefined on error.
 *   - Device buffers (Q, K, V, out, lse, Q_S, scores, head_scores, order, workspace) are
 *     owned by the caller and must stay alive until the work enqueued on `stream`
 *     completes.  Host arrays (segment_offsets, seg_ptr, doc_offsets, doc_ptr) are read
 *     only during the call.  The library keeps no per-call device state; it owns only a
 *     small pool of pinned host staging buffers for uploading the work plan.
 *   - Every compute call only enqueues work on `stream` (hipStream_t; 0 = null stream).
 *     The calling thread's current HIP device must be the stream's device.
 *   - Tensors are token-major and packed over all prompts ("THD"), bf16 = IEEE bfloat16
 *     bit patterns, contiguous, 16-byte aligned base pointers.
 *   - Supported: head_dim in {64, 128}; num_q_heads % num_kv_heads == 0 with
 *     G = num_q_heads / num_kv_heads in {1, 2, 4, 8}; query head h reads KV head h / G;
 *     num_q_heads * head_dim <= 65536 (512 query heads at d = 128); total_tokens <= 2^30 and
 *     total_tokens * num_kv_heads * head_dim * 2 < 2^32 (K and V each below 4 GiB: the attention
 *     kernel addresses them with 32-bit offsets); an attention plan of fewer than 2^21 work
 *     items (row tiles of 128 (token, head) rows plus the query's split-key chunks: far beyond
 *     what K and V below 4 GiB allow, except with very many one-token segments); others:
 *     BR_ERR_UNSUPPORTED.
 */
#ifndef BLOCKRANK_H
#define BLOCKRANK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BR_OK = 0,
  BR_ERR_INVALID_ARG = 1,  /* malformed sizes, tables or pointers */
  BR_ERR_UNSUPPORTED = 2,  /* well-formed but outside the supported shapes */
  BR_ERR_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_bytes */
  BR_ERR_HIP = 4           /* a HIP runtime call failed */
} br_status;

typedef struct {
  int32_t num_prompts;   /* B >= 1 */
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv, divides Hq */
  int32_t head_dim;      /* d: 64 or 128 */
  int64_t total_tokens;  /* T = sum of prompt lengths = last segment offset */
} br_dims;

/*
 * Segment table (host int32).  Prompt b owns
 *   segment_offsets[seg_ptr[b] .. seg_ptr[b+1]) = {s, s+p, s+p+l_1, ..., s+p+D, s+L}
 * i.e. N_b + 3 absolute token offsets, N_b >= 1: segment 0 is the instruction (p >= 0
 * tokens, may be empty), the last segment is the final query (q >= 1 tokens), the ones
 * between are the N_b documents (each l_k >= 1 token).  Prompts are contiguous:
 * segment_offsets[0] == 0, prompt b+1 starts where prompt b ends, and the last offset
 * equals dims->total_tokens.  seg_ptr is int32[B + 1] with seg_ptr[0] == 0.
 */

/* Bytes of device workspace br_attn_fwd needs for this table (plan + split-key partials). */
br_status br_attn_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets,
                                  const int32_t* seg_ptr, size_t* bytes);

/*
 * Block-sparse prefill attention for one layer.
 *   Q    device bf16 [T, Hq, d]      K, V  device bf16 [T, Hkv, d]
 *   out  device bf16 [T, Hq, d]      every row is written (no row has an empty key set:
 *                                    each token may read itself)
 *   lse  device fp32 [T, Hq] or NULL natural-log log-sum-exp of the scaled logits per row
 *   softmax_scale  <= 0 selects 1/sqrt(d)
 *   workspace      device, >= br_attn_workspace_bytes(), 256-byte aligned
 * Arithmetic: bf16 operands, fp32 accumulation and softmax statistics, probabilities
 * rounded to bf16 before the P.V product, output rounded to nearest even bf16.
 */
br_status br_attn_fwd(const br_dims* dims, const void* Q, const void* K, const void* V,
                      const int32_t* segment_offsets, const int32_t* seg_ptr, void* out,
                      float* lse, float softmax_scale, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * The same attention with BlockSearch's additive sink ("Can Language Models Actually Retrieve
 * In-Context?", section 5.1 "Length-aware softmax", and its appendix note on the sink): the
 * constant exp(sink) is appended to every row's softmax denominator, so
 *   out = softmax(s) V * sigma(lse - sink),   s the scaled logits, lse their log-sum-exp,
 * the gate sigma(lse - b_L) the note describes (b_L one scalar per layer, supplied by the
 * caller).  sink = -INFINITY gives br_attn_fwd's output bit for bit; NaN is rejected
 * (BR_ERR_INVALID_ARG).  lse (if non-NULL) is the plain log-sum-exp, without the sink.  Other
 * arguments, workspace size and errors as for br_attn_fwd.
 */
br_status br_attn_fwd_sink(const br_dims* dims, const void* Q, const void* K, const void* V,
                           const int32_t* segment_offsets, const int32_t* seg_ptr, void* out,
                           float* lse, float softmax_scale, float sink, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * br_attn_fwd, plus timing: records `kernel_start` on `stream` immediately before the main
 * attention kernel is enqueued and `kernel_stop` immediately after it (the split-key merge
 * kernel, if any, follows `kernel_stop`).  Either event may be NULL.  For measuring the
 * attention kernel's own duration with hipEventElapsedTime; results are identical to
 * br_attn_fwd.
 */
br_status br_attn_fwd_timed(const br_dims* dims, const void* Q, const void* K, const void* V,
                            const int32_t* segment_offsets, const int32_t* seg_ptr, void* out,
                            float* lse, float softmax_scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream, hipEvent_t kernel_start,
                            hipEvent_t kernel_stop);

/*
 * br_attn_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, bit for bit,
 * with no workspace argument.  Its workspace is a device array inside the library of
 * BR_NOALLOC_SCRATCH_BYTES bytes per GPU, held until the process ends; segment tables whose
 * br_attn_workspace_bytes exceeds it return BR_ERR_UNSUPPORTED.  The plan is copied from
 * pageable host memory with hipMemcpyAsync; nothing is allocated (no hipMalloc, hipFree or
 * pinned staging).  Every call on a GPU uses that GPU's one array: calls that overlap on one
 * GPU (two streams, or a second host thread) race and must be serialised by the caller.
 * Other arguments, rules and errors as br_attn_fwd.
 */
#define BR_NOALLOC_SCRATCH_BYTES (32u << 20)
br_status br_attn_fwd_noalloc(const br_dims* dims, const void* Q, const void* K, const void* V,
                              const int32_t* segment_offsets, const int32_t* seg_ptr, void* out,
                              float* lse, float softmax_scale, hipStream_t stream);

/*
 * Document spans (host int32).  Prompt b owns doc_offsets[doc_ptr[b] .. doc_ptr[b+1]),
 * N_b + 1 increasing absolute token offsets (normally segment_offsets[1 .. N_b+2) of that
 * prompt); document k of prompt b is [doc_offsets[doc_ptr[b]+k], doc_offsets[doc_ptr[b]+k+1]).
 * Its score is stored at index doc_ptr[b] - b + k.  Spans must lie inside [0, T).
 */
br_status br_doc_scores_workspace_bytes(const br_dims* dims, int32_t n_signal,
                                        const int32_t* doc_offsets, const int32_t* doc_ptr,
                                        size_t* bytes);

/*
 * Attention-mass document scores.
 *   Q_S          device bf16 [B, n_signal, Hq, d]: the signal-carrier query rows
 *   K            device bf16 [T, Hkv, d] (the same layer's keys as the attention)
 *   scores       device fp32 [sum_b N_b]: s_k = (1/Hq) sum_h sum_i sum_{j in d_k} alpha'_{ihj}
 *   head_scores  device fp32 [Hq, sum_b N_b] (per-head signal-row sums) or NULL
 *   softmax_scale <= 0 selects 1/sqrt(d)
 * n_signal in [1, 64]; sum_k s_k = n_signal per prompt up to rounding.
 */
br_status br_doc_scores(const br_dims* dims, const void* Q_S, int32_t n_signal, const void* K,
                        const int32_t* doc_offsets, const int32_t* doc_ptr, float* scores,
                        float* head_scores, float softmax_scale, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * Per-prompt ranking.  scores: device fp32 [sum_b N_b] laid out as br_doc_scores writes
 * them; doc_ptr: host int32[B + 1] as above (only differences are used: N_b =
 * doc_ptr[b+1] - doc_ptr[b] - 1).  order: device int32 [sum_b N_b]; for prompt b, entries
 * doc_ptr[b]-b .. +N_b hold local document indices in descending score order, ties to the
 * lower index; NaN scores rank as -infinity.  N_b <= 65,536 (BR_ERR_UNSUPPORTED above: the
 * exact counting sort does N_b^2 comparisons per prompt).
 */
br_status br_sort_docs(const float* scores, const int32_t* doc_ptr, int32_t num_prompts,
                       int32_t* order, hipStream_t stream);

/*
 * Top-B routed attention (BlockSearch, section 5.1 "Document-level sparse attention": only the
 * top-B documents by score take part in attention from the routing layer on).  Prompt b keeps
 * the documents keep[keep_ptr[b] .. keep_ptr[b + 1]) (HOST int32 local indices 0..N_b-1, each at
 * most once, any order; keep_ptr: HOST int32[B + 1], keep_ptr[0] == 0).  Instruction rows and
 * kept documents' rows are computed as in br_attn_fwd; dropped documents' rows are not
 * computed (their out and lse rows are left untouched); final-query rows read the instruction
 * and the kept documents unmasked and the query causally.  Keeping every document gives
 * exactly br_attn_fwd's result.  Other arguments and rules as br_attn_fwd.
 */
br_status br_attn_routed_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets,
                                         const int32_t* seg_ptr, const int32_t* keep_ptr,
                                         const int32_t* keep, size_t* bytes);
br_status br_attn_routed_fwd(const br_dims* dims, const void* Q, const void* K, const void* V,
                             const int32_t* segment_offsets, const int32_t* seg_ptr,
                             const int32_t* keep_ptr, const int32_t* keep, void* out, float* lse,
                             float softmax_scale, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * The whole hot path in one call: br_attn_fwd, br_doc_scores and br_sort_docs on the same
 * inputs, with both work plans uploaded in one copy.  Arguments, layouts and rules as in those
 * three calls (softmax_scale serves the attention and the readout); outputs are bit-identical to
 * theirs.  workspace: >= br_rank_workspace_bytes(), 16-byte aligned.  br_rank_prompts_timed
 * also records kernel_start / kernel_stop (hipEvent_t, may be NULL) on `stream` immediately
 * around the attention kernel.
 * Streams: for batches of at least 24,576 tokens (timed or not), the readout and rank,
 * which read only the inputs, run on a stream the library owns (one per device, default
 * priority, created on first use and kept until the process ends), forked from `stream` after
 * the plan upload and joined back into it; work enqueued on `stream` afterwards, and a
 * synchronisation of `stream`, see every output.  Otherwise everything runs on `stream`.
 * Plans: the library keeps the last four validated and scheduled plans (process lifetime) and
 * reuses one when a call's dims, n_signal and four host tables equal an entry's element by
 * element on the same device; the host arrays are still read during the call only.  A new plan
 * is uploaded into the workspace.  The first call that reuses a plan copies its image (a few
 * hundred KB at 100K tokens) into device memory the library allocates, with a blocking copy and
 * a device synchronisation; that call and later ones read the plan there and upload nothing.
 * Dropping a plan from the four frees its copy after a device synchronisation.
 */
br_status br_rank_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                                  int32_t n_signal, const int32_t* doc_offsets, const int32_t* doc_ptr,
                                  size_t* bytes);
br_status br_rank_prompts(const br_dims* dims, const void* Q, const void* K, const void* V, const void* Q_S,
                          int32_t n_signal, const int32_t* segment_offsets, const int32_t* seg_ptr,
                          const int32_t* doc_offsets, const int32_t* doc_ptr, void* out, float* lse,
                          float* scores, float* head_scores, int32_t* order, float softmax_scale,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);
br_status br_rank_prompts_timed(const br_dims* dims, const void* Q, const void* K, const void* V,
                                const void* Q_S, int32_t n_signal, const int32_t* segment_offsets,
                                const int32_t* seg_ptr, const int32_t* doc_offsets, const int32_t* doc_ptr,
                                void* out, float* lse, float* scores, float* head_scores, int32_t* order,
                                float softmax_scale, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, hipEvent_t kernel_start, hipEvent_t kernel_stop);

/*
 * Block-sparse attention with the rotary embedding of Q applied inside the attention kernel
 * (BlockRank summary, section 3.4 "Permutation-invariant position embeddings"): Q is given
 * unrotated and each work item rotates its Q rows in registers as it reads them, with cos/sin
 * from a table of the prompts' distinct positions (built on the device by the rotation kernel's
 * own code, so the rotated values equal br_rope_fwd's); K must already be rotated with the same
 * rule (br_rope_fwd with Q = NULL).  rope_theta, query_pos0, docs_after_instruction and
 * interleaved as for br_rope_fwd.  Output: bit-identical to br_rope_fwd on Q followed by
 * br_attn_fwd.  workspace: >= br_attn_fwd_rope_workspace_bytes() (the attention plan plus the
 * table: (distinct positions) x d x 4 bytes), 256-byte aligned.  Errors as br_attn_fwd and
 * br_rope_fwd.
 */
br_status br_attn_fwd_rope_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets,
                                           const int32_t* seg_ptr, int32_t query_pos0,
                                           int32_t docs_after_instruction, size_t* bytes);
br_status br_attn_fwd_rope(const br_dims* dims, const void* Q, const void* K, const void* V,
                           const int32_t* segment_offsets, const int32_t* seg_ptr, void* out, float* lse,
                           float softmax_scale, float rope_theta, int32_t query_pos0,
                           int32_t docs_after_instruction, int32_t interleaved, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * Query-only attention over a cached corpus ("prefill once, score many queries"; BlockSearch,
 * section 3.2: the query block attends over the full corpus and causally to itself).
 * The key/value token axis holds the corpus [0, corpus_len) (e.g. an instruction and its
 * documents, already prefilled) followed by dims->num_prompts queries; query b owns tokens
 * [query_offsets[b], query_offsets[b + 1]) and each of its rows reads every corpus key
 * unmasked plus its own query's keys up to itself.  Corpus rows are not computed.
 *   query_offsets: HOST int32[num_prompts + 1], query_offsets[0] == corpus_len, strictly
 *                  increasing, last == dims->total_tokens (= corpus_len + query tokens).
 *   Q, out: device bf16 [total_tokens - corpus_len, Hq, d] (query rows only, in token order);
 *   K, V:   device bf16 [total_tokens, Hkv, d];  lse: device fp32 [total_tokens - corpus_len, Hq]
 *           or NULL.  Other rules (scale, alignment, workspace, errors) as br_attn_fwd.
 */
br_status br_query_attn_workspace_bytes(const br_dims* dims, int32_t corpus_len, const int32_t* query_offsets,
                                        size_t* bytes);
br_status br_query_attn_fwd(const br_dims* dims, const void* Q, const void* K, const void* V, int32_t corpus_len,
                            const int32_t* query_offsets, void* out, float* lse, float softmax_scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Host-only introspection of the attention work plan (no HIP call).  Writes up to
 * `capacity` work items of 8 int32 each, {row0, row_limit, a_start, a_end, b_start, b_end,
 * partial_slot, tile_count}: the row tile starts at token row0 and covers the tokens
 * [row0, min(row0 + rows_per_tile, row_limit)) of every query head of a KV group; it reads
 * keys [a_start, a_end) unmasked and [b_start, b_end) causally (key <= row token).
 * partial_slot >= 0 marks one chunk of a split query tile.  The list is the same for
 * every KV head.  *n_items receives the item count, *rows_per_tile the token rows per tile.
 */
br_status br_attn_plan_items(const br_dims* dims, const int32_t* segment_offsets,
                             const int32_t* seg_ptr, int32_t* items, int64_t capacity,
                             int64_t* n_items, int32_t* rows_per_tile);

/*
 * Host-only introspection of the persistent schedule (no HIP call) that br_attn_fwd builds
 * for a device with `workgroups` persistent workgroup slots (compute units x 2 on gfx950).
 * Workgroup w of each KV head runs the items sched[ranges[w] .. ranges[w+1]) in that order;
 * `sched` (8 int32 per item, as br_attn_plan_items) is a permutation of the plan's item list.
 * Buffers: sched holds `capacity` items, ranges holds `ranges_capacity` int32; each is written
 * only if large enough (n_items items, wg_per_head + 1 offsets), else only the counts are.
 * *n_items and *wg_per_head receive the counts.  workgroups < 1 is BR_ERR_INVALID_ARG.
 */
br_status br_attn_plan_schedule(const br_dims* dims, const int32_t* segment_offsets,
                                const int32_t* seg_ptr, int32_t workgroups, int32_t* sched,
                                int64_t capacity, int32_t* ranges, int64_t ranges_capacity,
                                int64_t* n_items, int32_t* wg_per_head);

/*
 * Backward of br_attn_fwd (BlockRank summary, section 3.4: the auxiliary loss's gradient flows
 * back through this attention).  For the upstream gradient dO, with P = softmax over the allowed
 * keys of scale * Q K^T (recomputed from lse, never stored):
 *   dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),  dQ = scale * dS K,  dK = scale * dS^T Q,
 * where grouped query heads add into their KV head's dK and dV.  Only allowed pairs are visited.
 *   Q, O, dO: device bf16 [total_tokens, Hq, d];  K, V: device bf16 [total_tokens, Hkv, d];
 *   lse: device fp32 [total_tokens, Hq], natural-log log-sum-exp from br_attn_fwd with the same
 *        softmax_scale;  O: br_attn_fwd's output.
 *   dQ: device fp32 [total_tokens, Hq, d];  dK, dV: device fp32 [total_tokens, Hkv, d]; every
 *       element is written.
 *   Segment tables, scale, alignment and errors as br_attn_fwd; workspace as sized by
 *   br_attn_bwd_workspace_bytes (it also holds rowsum(dO * O), -lse * log2(e) and split partial
 *   sums).
 * Arithmetic: P and dS in fp32, rounded to bf16 for the P^T dO, dS K and dS^T Q products,
 * fp32 accumulation; split partial sums are added in a fixed order (deterministic).
 */
br_status br_attn_bwd_workspace_bytes(const br_dims* dims, const int32_t* segment_offsets,
                                      const int32_t* seg_ptr, size_t* bytes);
br_status br_attn_bwd(const br_dims* dims, const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* lse, const int32_t* segment_offsets,
                      const int32_t* seg_ptr, float* dQ, float* dK, float* dV, float softmax_scale,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Host-only introspection of the backward's key-major plan (no HIP call).  Writes up to
 * `capacity` items of 8 int32 each, {k0, k_limit, c0, c1, u0, u1, partial_slot, row_tokens}:
 * keys [k0, k_limit) of one segment, read causally (row token >= key) by rows [c0, c1) and
 * unmasked by rows [u0, u1); partial_slot >= 0 marks one chunk of a split row range.
 * *n_items and *n_slots receive the counts; items is written only if capacity suffices.
 */
br_status br_attn_bwd_plan_items(const br_dims* dims, const int32_t* segment_offsets,
                                 const int32_t* seg_ptr, int32_t* items, int64_t capacity,
                                 int64_t* n_items, int32_t* n_slots);

/*
 * InfoNCE auxiliary loss on the readout scores (BlockRank summary, section 3.4 "auxiliary
 * contrastive loss"; blog, attention supervision): per prompt b with documents k = 0..N_b-1,
 *   loss[b] = -log(exp(s_gold / tau) / sum_k exp(s_k / tau)),
 *   dscores[k] = d(sum_b loss[b]) / ds_k = (softmax(s / tau)_k - [k == gold]) / tau.
 *   scores, dscores: device fp32 [sum_b N_b] (br_doc_scores order);  loss: device fp32 [B].
 *   doc_ptr: HOST int32[B + 1] as for br_doc_scores;  gold: HOST int32[B], 0 <= gold[b] < N_b.
 *   tau > 0 and finite (the pages use 0.05); N_b <= 65,536.  fp32 arithmetic.
 *   workspace: device, >= br_infonce_workspace_bytes(B), 16-byte aligned.
 */
br_status br_infonce_workspace_bytes(int32_t num_prompts, size_t* bytes);
br_status br_infonce(const float* scores, const int32_t* doc_ptr, int32_t num_prompts, const int32_t* gold,
                     float tau, float* loss, float* dscores, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * Backward of br_doc_scores: the gradient of sum_k dscores_k s_k with respect to Q_S and K
 * (BlockRank summary, section 3.4: the auxiliary loss's gradient flows back through the
 * readout's attention).  With alpha the readout softmax over the prompt's document tokens of
 * z = scale Q_S K^T and c_(i,h) = sum_k alpha-mass_(i,h,k) dscores_k:
 *   dz = alpha * (dscores_k(j) - c) / Hq,  dQ_S = scale * dz K,  dK = scale * dz^T Q_S
 * (query heads of a group add into their KV head).
 *   Q_S, K, doc_offsets, doc_ptr, n_signal, softmax_scale: as for br_doc_scores.
 *   dscores: device fp32 [sum_b N_b];  dQ_S: device fp32 [B, n_signal, Hq, d] (fully written);
 *   dK: device fp32 [total_tokens, Hkv, d]: rows of document tokens are written
 *       (accumulate == 0) or added to (accumulate == 1, e.g. onto br_attn_bwd's dK); other rows
 *       are not touched.
 *   n_signal * (Hq / Hkv) <= 64 (BR_ERR_UNSUPPORTED otherwise).
 *   workspace: device, >= br_doc_scores_bwd_workspace_bytes(), 16-byte aligned.
 * Arithmetic: alpha and dz in fp32, dz rounded to bf16 for the two MFMA products, fp32 sums; the
 * per-group dQ_S partials are added in a fixed order (deterministic).
 */
br_status br_doc_scores_bwd_workspace_bytes(const br_dims* dims, int32_t n_signal, const int32_t* doc_offsets,
                                            const int32_t* doc_ptr, size_t* bytes);
br_status br_doc_scores_bwd(const br_dims* dims, const void* Q_S, int32_t n_signal, const void* K,
                            const int32_t* doc_offsets, const int32_t* doc_ptr, const float* dscores,
                            float* dQ_S, float* dK, int32_t accumulate, float softmax_scale, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * SSMax logit factor (BlockSearch, section 5.1, length-aware softmax): SSMax multiplies the
 * pre-softmax scores q.k / sqrt(d) by s * ln N, N the number of documents of the prompt.  Writes
 * *scale = s * ln(n_docs) / sqrt(head_dim), the value to pass as softmax_scale to
 * br_attn_fwd / br_attn_routed_fwd / br_query_attn_fwd and br_doc_scores for that prompt (the
 * factor is per call, so a batch shares one N).  Host only.  n_docs < 2 is BR_ERR_INVALID_ARG
 * (ln 1 = 0 would zero every logit, which softmax_scale cannot express: 0 selects 1/sqrt(d));
 * s must be finite and positive; head_dim >= 1.
 */
br_status br_ssmax_softmax_scale(float s, int32_t n_docs, int32_t head_dim, float* scale);

/*
 * Rotary position embedding with permutation-invariant position ids (BlockRank summary,
 * section 3.4 "Permutation-invariant position embeddings"; BlockSearch, section 3.2).
 * Positions within prompt b (segments as for br_attn_fwd): instruction token i -> i; token j
 * of any document -> j + (docs_after_instruction ? instruction length : 0); final-query token
 * i -> query_pos0 + i.  BlockRank's rule is docs_after_instruction = 1, query_pos0 = 8192;
 * BlockSearch's is docs_after_instruction = 0, query_pos0 = 300.
 * Rotation (RoFormer): pair k of every head vector turns by pos * rope_theta^(-2k/d),
 *   a' = a cos - b sin,  b' = a sin + b cos,
 * with pairs (k, k + d/2) when interleaved == 0 (split halves, the GPT-NeoX / Mistral layout)
 * or (2k, 2k + 1) when interleaved == 1.  The angle is reduced in fp64, the rotation runs in
 * fp32 and the result is rounded to bf16 (nearest even).
 *   Q, Q_out: device bf16 [total_tokens, Hq, d];  K, K_out: device bf16 [total_tokens, Hkv, d].
 *   Q_out may equal Q and K_out may equal K (in place).  Q and Q_out may both be NULL, or K and
 *   K_out, but not all four.  16-byte aligned.
 *   rope_theta: finite, > 0 (the base is a model parameter; it is not on the pages).
 *   query_pos0 >= 0; query positions must fit in int32.
 *   workspace: device, >= br_rope_workspace_bytes(), 16-byte aligned, owned by the caller;
 *   it holds the uploaded position runs while the enqueued kernel runs.
 * Errors as in the conventions above; nothing is enqueued on error.
 */
br_status br_rope_workspace_bytes(const br_dims* dims, const int32_t* seg_ptr, size_t* bytes);
br_status br_rope_fwd(const br_dims* dims, const void* Q, const void* K, void* Q_out, void* K_out,
                      const int32_t* segment_offsets, const int32_t* seg_ptr, float rope_theta,
                      int32_t query_pos0, int32_t docs_after_instruction, int32_t interleaved,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same rotation for the readout's signal rows: Q_S, Q_S_out device bf16
 * [num_prompts, n_signal, Hq, d]; row s of prompt b is the prompt's query token
 * q_b - n_signal + s and sits at position query_pos0 + q_b - n_signal + s.  Each query must
 * hold at least n_signal tokens.  Workspace as br_rope_workspace_bytes.
 */
br_status br_rope_signal_fwd(const br_dims* dims, const void* Q_S, void* Q_S_out, int32_t n_signal,
                             const int32_t* segment_offsets, const int32_t* seg_ptr, float rope_theta,
                             int32_t query_pos0, int32_t interleaved, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/*
 * Host-only (no HIP call): the position id of every token under the rule above, written to the
 * host array positions[total_tokens] (capacity >= total_tokens).
 */
br_status br_rope_positions(const br_dims* dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                            int32_t query_pos0, int32_t docs_after_instruction, int32_t* positions,
                            int64_t capacity);

const char* br_status_string(br_status status);
const char* br_last_error(void);
const char* br_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLOCKRANK_H */
