// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace br {

struct AttnLaunch {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* V;
  uint16_t* O;
  float* lse;
  const AttnItem* items;    // device copy of the plan's items
  const int32_t* ranges;    // device copy of the per-workgroup item ranges [wg_per_head + 1]
  const MergeItem* merges;  // device copy of the plan's merges
  float* part_o;
  float* part_ml;
  int64_t n_items, n_merges;
  int wg_per_head;
  int num_q_heads, num_kv_heads, head_dim;
  float scale_log2;         // softmax scale * log2(e)
  int q_row_base = 0;       // token index of Q/O/lse row 0 (the corpus length for query-only runs)
  float sink_log2 = -__builtin_inff();  // additive sink b * log2(e); -inf: none
  int rope = 0;                      // 0 none; 1 / 2: rotate Q in the kernel (split / adjacent pairs)
  const float* rope_cs = nullptr;    // [table rows][D/2][cos, sin]
  const int32_t* item_pidx = nullptr;  // per scheduled item: table row of its first token
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;  // optional, recorded around the main kernel
  bool defer_merge = false;  // leave the split-key merge to launch_merge_doc_scores
};
hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream);

struct ScoreLaunch {
  const uint16_t* Q_S;
  const uint16_t* K;
  const ScoreItem* items;
  const int32_t* doc_offsets;   // device copy
  const int32_t* prompt_base;   // device copy, [B + 1] score index of each prompt's first document
  float2* ml;                   // [n_docs, n_signal * Hq] partial (max, sum)
  float* scores;
  float* head_scores;
  int64_t n_items;
  int num_prompts, num_q_heads, num_kv_heads, head_dim, n_signal, row_blocks, n_docs;
  float scale_log2;
};
hipError_t launch_doc_scores(const ScoreLaunch& a, hipStream_t stream);
// The readout's per-document (m_k, e_k) and per-row (M, 1/Z) only (rowstat at ml + n_docs * RT).
hipError_t launch_doc_stats(const ScoreLaunch& a, hipStream_t stream);
// The readout with the attention's deferred split-key merge (launch_attn with defer_merge) in the
// launch of its partial kernel; same results as launch_attn followed by launch_doc_scores.
hipError_t launch_merge_doc_scores(const AttnLaunch& attn, const ScoreLaunch& a, hipStream_t stream);

struct DocBwdLaunch {
  const uint16_t* Q_S;
  const uint16_t* K;
  const ScoreItem* items;
  const int32_t* doc_offsets;
  const int32_t* prompt_base;
  const int32_t* prompt_items;
  const float2* ml;
  const float2* rowstat;
  float* center;
  const float* dscores;
  float* dK;
  float* part;
  float* dQ_S;
  int64_t n_items;
  int num_prompts, num_q_heads, num_kv_heads, head_dim, n_signal, row_blocks, accumulate;
  float scale;
};
hipError_t launch_doc_bwd(const DocBwdLaunch& a, hipStream_t stream);
hipError_t launch_infonce(const float* scores, const int32_t* prompt_base, const int32_t* gold, float tau,
                          int num_prompts, float* loss, float* dscores, hipStream_t stream);

constexpr int kSortMaxDocs = 65536;  // documents per prompt (the counting sort is O(N^2) per prompt)
constexpr int kSortPromptsPerLaunch = 256;
hipError_t launch_sort_docs(const float* scores, const int32_t* prompt_base, int num_prompts, int32_t* order,
                            hipStream_t stream);

struct BwdLaunch {
  const uint16_t *Q, *K, *V, *O, *dO;
  const float* lse;          // [T, Hq] natural-log log-sum-exp from the forward
  float *dQ, *dK, *dV;       // fp32 outputs
  float* dvec;               // [T, Hq] workspace: rowsum(dO * O)
  float* nlse2;              // [T, Hq] workspace: -lse * log2(e)
  const AttnItem* items;     // device copies of the forward plan's items and merges
  const MergeItem* merges;
  float* part_dq;
  const KvItem* kv_items;    // device copies of the key-major items and merges
  const KvMerge* kv_merges;
  float* part_dkv;
  int64_t n_items, n_merges, n_kv_items, n_kv_merges, total_tokens;
  int kv_slots, num_q_heads, num_kv_heads, head_dim;
  float scale;
};
hipError_t launch_attn_bwd(const BwdLaunch& a, hipStream_t stream);

struct RopeLaunch {
  const uint16_t* q;        // [rows, q_heads, head_dim] or nullptr (q_heads == 0)
  uint16_t* q_out;          // may equal q
  const uint16_t* k;        // [rows, k_heads, head_dim] or nullptr (k_heads == 0)
  uint16_t* k_out;          // may equal k
  const int32_t* run_start;  // device copies of the plan's runs
  const int32_t* run_pos0;
  const double* inv_freq;
  int64_t rows;
  int n_runs, q_heads, k_heads, head_dim;
  bool adjacent;            // pairs (2k, 2k+1) instead of (k, k + d/2)
};
hipError_t launch_rope(const RopeLaunch& a, hipStream_t stream);
// cos/sin table of the attention's fused Q rotation ([rows][head_dim / 2] pairs of fp32).
hipError_t launch_rope_table(const int32_t* iv_pos0, const int32_t* iv_off, int n_iv, int64_t rows, int head_dim,
                             const double* inv_freq, float* table, hipStream_t stream);

}  // namespace br
