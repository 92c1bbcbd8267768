// Host-side validation and work planning for the BlockRank attention and readout kernels.
// Pure C++ (no HIP calls), so it is unit-testable without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "blockrank.h"

namespace br {

// Attention tiling shared by the planner and the kernels.
constexpr int kRowsPerWave = 32;                  // one 32x32 MFMA block of query rows per wave
constexpr int kWaves = 4;                         // waves per workgroup
constexpr int kRowsPerTile = kRowsPerWave * kWaves;  // 128 (token, head) rows per work item
constexpr int kKeyTile = 64;                      // keys staged in LDS per step
constexpr int kAttnWgPerCu = 2;                   // persistent attention workgroups per CU
constexpr int kMaxAttnWgPerHead = 4096;           // bound on workgroups sharing one KV head
// Bound on the items of one attention plan: the kernel packs an item index into the upper bits of
// a 32-bit tile code (21 bits above 10 bits of key count and flags).
constexpr int64_t kMaxAttnItems = int64_t(1) << 21;
constexpr int kMaxHeadsTimesDim = 65536;          // bound on num_q_heads * head_dim (512 heads at d = 128)

inline int tokens_per_tile(int group) { return kRowsPerTile / group; }

// One attention work item; the same list is run for every KV head.
// Rows: tokens [row0, min(row0 + TM, row_limit)) of the G query heads of the KV head.
// Keys: [a_start, a_end) read unmasked, then [b_start, b_end) read causally.
struct AttnItem {
  int32_t row0, row_limit;
  int32_t a_start, a_end;
  int32_t b_start, b_end;
  int32_t slot;    // -1: write the output rows; >= 0: write split-key partials to this slot
  int32_t ntiles;  // key tiles visited (for scheduling and accounting)
};
static_assert(sizeof(AttnItem) == 32, "AttnItem is read as two int4 by the kernel");

// One split query tile: merge partial slots [slot0, slot0 + nslots) into rows.
struct MergeItem {
  int32_t row0, row_limit, slot0, nslots;
};

struct AttnPlan {
  int group = 1;             // G = Hq / Hkv
  int rows_per_tile = 128;   // TM tokens per tile
  int key_tile = kKeyTile;
  int chunk_keys = 0;        // split-key chunk length for query rows
  std::vector<AttnItem> items;
  std::vector<MergeItem> merges;
  int32_t n_slots = 0;       // partial slots per KV head
  // Persistent schedule: workgroup w of a KV head runs sched[ranges[w] .. ranges[w+1]), a
  // permutation of `items` (which stays in the planner's time order).
  int wg_per_head = 1;
  std::vector<AttnItem> sched;
  std::vector<int32_t> ranges;
  // workspace layout (bytes from the workspace base)
  size_t off_items = 0, off_ranges = 0, off_merges = 0, off_part_o = 0, off_part_ml = 0, total_bytes = 0;
};

struct ScoreItem {
  int32_t prompt;      // prompt index b
  int32_t d0, d1;      // global indices into doc_offsets: documents [d0, d1) (d1 - d0 >= 1)
  int32_t score_base;  // scores index of document d0
};

struct ScorePlan {
  int group = 1;
  int n_signal = 1;
  int rows_per_kv = 1;   // n_signal * G
  int row_blocks = 1;    // ceil(rows_per_kv / 32)
  int32_t n_docs = 0;    // sum_b N_b
  std::vector<ScoreItem> items;
  std::vector<int32_t> prompt_score_base;  // [B + 1]
  size_t off_items = 0, off_doc_offsets = 0, off_prompt_base = 0, off_ml = 0, total_bytes = 0;
};

// Backward of the attention.  dQ is query-major over the forward plan's items (split query
// tiles write fp32 partials summed afterwards); dK and dV are key-major: an item holds keys
// [k0, k_limit) of one segment (at most kBwdKeyTile) and the rows that read them, [c0, c1)
// causally (row token >= key) and [u0, u1) unmasked.  Long unmasked row ranges (the rows that
// read the instruction) are split into chunks of kBwdRowChunk tokens with fp32 partials.
constexpr int kBwdKeyTile = 64;
constexpr int kBwdRowChunk = 4096;
// Documents whose key tiles the dK/dV pass runs together: groups close once they hold this many
// document tokens, so that the rows the group's tiles read (Q and dO: 2048 tokens x 4 heads x
// 512 B = 4 MB at 4 query heads per KV head and d = 128) stay in the L2 of the XCD serving the
// head between the tiles that re-read them.
constexpr int kBwdGroupTokens = 2048;
struct KvItem {
  int32_t k0, k_limit, c0, c1, u0, u1, slot, rows;  // rows: row tokens visited (for accounting)
};
static_assert(sizeof(KvItem) == 32, "KvItem is read as two int4 by the kernel");
struct KvMerge {
  int32_t k0, k_limit, slot0, nslots;
};
struct BwdPlan {
  AttnPlan fwd;
  std::vector<KvItem> kv_items;
  std::vector<KvMerge> kv_merges;
  int32_t kv_slots = 0;
  size_t off_items = 0, off_merges = 0, off_part_dq = 0, off_kv_items = 0, off_kv_merges = 0, off_part_dkv = 0,
         off_dvec = 0, total_bytes = 0;
};

// Backward of the readout: the forward score plan (its items stream each document's keys once)
// plus, per prompt, the range of its items (for summing the per-item dQ_S partials).  Signal
// rows per KV head (n_signal * G) are limited to kDocBwdMaxRows.
constexpr int kDocBwdMaxRows = 64;
constexpr int kInfoNceMaxDocs = 65536;
struct DocBwdPlan {
  ScorePlan fwd;
  std::vector<int32_t> prompt_items;  // [B + 1]
  size_t off_prompt_items = 0, off_center = 0, off_part = 0, total_bytes = 0;
};

// Rotary embedding runs: rows [start[r], start[r + 1]) take positions pos0[r] + (row - start[r]).
// Runs are non-empty and ascending; start has n_runs + 1 entries, the last being the row count.
struct RopePlan {
  std::vector<int32_t> start;
  std::vector<int32_t> pos0;
  std::vector<double> inv_freq;  // theta^(-2k/d), k = 0 .. d/2 - 1
  int64_t rows = 0;
  size_t off_start = 0, off_pos0 = 0, off_freq = 0, total_bytes = 0;
};

// Status plus message; the API layer stores the message in the thread-local error slot.
struct Error {
  br_status status = BR_OK;
  std::string msg;
  bool ok() const { return status == BR_OK; }
};

Error validate_dims(const br_dims* dims);
Error validate_segments(const br_dims& dims, const int32_t* segment_offsets, const int32_t* seg_ptr);
Error build_attn_plan(const br_dims& dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                      AttnPlan* plan);
// Query-only plan over a cached corpus: dims.num_prompts queries; query b owns key/value tokens
// [query_offsets[b], query_offsets[b + 1]) after the corpus [0, corpus_len) and reads the whole
// corpus unmasked plus its own tokens causally.
Error validate_queries(const br_dims& dims, int32_t corpus_len, const int32_t* query_offsets);
Error build_query_plan(const br_dims& dims, int32_t corpus_len, const int32_t* query_offsets, AttnPlan* plan);
// Top-B routing: prompt b keeps documents keep[keep_ptr[b] .. keep_ptr[b + 1]) (local indices).
// Kept documents' rows are computed as in build_attn_plan; dropped documents' rows are not
// computed; query rows read the instruction and the kept documents unmasked, then themselves.
Error validate_keep(const br_dims& dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                    const int32_t* keep_ptr, const int32_t* keep);
Error build_routed_plan(const br_dims& dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                        const int32_t* keep_ptr, const int32_t* keep, AttnPlan* plan);
// Partition the item list over the persistent workgroups of each KV head.  `workgroups` = the
// device's persistent workgroup slots (CUs x kAttnWgPerCu); it shapes only the partition, never
// the items or the workspace size.  Calling it again re-partitions from `items`.
void schedule_attn_plan(int num_kv_heads, int workgroups, AttnPlan* plan);
// Relative cost of an item in the schedule (quarter key tiles).
int64_t attn_item_cost(const AttnItem& it);
Error validate_docs(const br_dims& dims, int32_t n_signal, const int32_t* doc_offsets,
                    const int32_t* doc_ptr);
Error build_score_plan(const br_dims& dims, int32_t n_signal, const int32_t* doc_offsets,
                       const int32_t* doc_ptr, ScorePlan* plan);

// Backward plan: the forward plan's items for dQ, key-major items for dK and dV, workspace layout.
Error build_bwd_plan(const br_dims& dims, const int32_t* segment_offsets, const int32_t* seg_ptr, BwdPlan* plan);

Error build_doc_bwd_plan(const br_dims& dims, int32_t n_signal, const int32_t* doc_offsets, const int32_t* doc_ptr,
                         DocBwdPlan* plan);
// InfoNCE over each prompt's scores: validates doc_ptr and gold; workspace [prompt bases | gold].
Error validate_infonce(int32_t num_prompts, const int32_t* doc_ptr, const int32_t* gold, float tau);
size_t infonce_workspace_bytes(int32_t num_prompts);

// Permutation-invariant positions: instruction token i at i; token j of a document at
// j + (docs_after_instruction ? instruction length : 0); query token i at query_pos0 + i.
Error validate_rope(const br_dims& dims, float rope_theta, int32_t query_pos0);
Error build_rope_plan(const br_dims& dims, const int32_t* segment_offsets, const int32_t* seg_ptr,
                      float rope_theta, int32_t query_pos0, int32_t docs_after_instruction, RopePlan* plan);
// Signal rows [B, n_signal]: row s of prompt b sits at the position of the prompt's query token
// q_b - n_signal + s.
Error build_rope_signal_plan(const br_dims& dims, int32_t n_signal, const int32_t* segment_offsets,
                             const int32_t* seg_ptr, float rope_theta, int32_t query_pos0, RopePlan* plan);
// Workspace for either plan: enough for one run per segment of the segment table.
size_t rope_workspace_bytes(int64_t n_runs, int head_dim);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace br
