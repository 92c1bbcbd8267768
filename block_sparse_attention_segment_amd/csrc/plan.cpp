// Validation of the segment / document tables and construction of the work plans.
//
// The attention plan realises the BlockRank token-type rules (BlockRank summary, section 3.4
// "Blockwise Structured Attention"; blog, block mask M) as a list of row tiles, each with at
// most two key ranges: an unmasked range (the instruction, or a chunk of everything before the
// final query) and a causal range (the tile's own segment up to its last row).  Only these
// ranges are ever visited, so no forbidden block is formed.  Key tiles of the causal range
// start at the segment start and key tiles of the instruction range at the prompt start, so a
// document's arithmetic does not depend on where the document sits in the prompt.
#include "plan.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <functional>
#include <utility>
#include <vector>

namespace br {
namespace {

Error fail(br_status s, const char* fmt, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b, c);
  return Error{s, buf};
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

Error validate_dims(const br_dims* dims) {
  if (!dims) return fail(BR_ERR_INVALID_ARG, "dims is NULL");
  if (dims->num_prompts < 1) return fail(BR_ERR_INVALID_ARG, "num_prompts must be >= 1 (got %lld)", dims->num_prompts);
  if (dims->num_q_heads < 1 || dims->num_kv_heads < 1)
    return fail(BR_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%lld, Hkv=%lld)", dims->num_q_heads, dims->num_kv_heads);
  if (dims->num_q_heads % dims->num_kv_heads)
    return fail(BR_ERR_INVALID_ARG, "num_q_heads (%lld) is not a multiple of num_kv_heads (%lld)", dims->num_q_heads,
                dims->num_kv_heads);
  int g = dims->num_q_heads / dims->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(BR_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %lld)", g);
  if (dims->head_dim <= 0) return fail(BR_ERR_INVALID_ARG, "head_dim must be positive (got %lld)", dims->head_dim);
  if (dims->head_dim != 64 && dims->head_dim != 128)
    return fail(BR_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %lld)", dims->head_dim);
  // Kernels address a tile of up to 128 token rows of all query heads with 32-bit byte offsets.
  if (int64_t(dims->num_q_heads) * dims->head_dim > kMaxHeadsTimesDim)
    return fail(BR_ERR_UNSUPPORTED, "num_q_heads * head_dim = %lld exceeds %lld",
                int64_t(dims->num_q_heads) * dims->head_dim, int64_t(kMaxHeadsTimesDim));
  if (dims->total_tokens < 1) return fail(BR_ERR_INVALID_ARG, "total_tokens must be >= 1 (got %lld)", dims->total_tokens);
  if (dims->total_tokens > (int64_t(1) << 30))
    return fail(BR_ERR_UNSUPPORTED, "total_tokens %lld exceeds 2^30", dims->total_tokens);
  // The attention kernel addresses K and V tiles with 32-bit byte offsets from the tensor base.
  if (dims->total_tokens * dims->num_kv_heads * dims->head_dim * 2 > int64_t(0xFFFFFFFFll))
    return fail(BR_ERR_UNSUPPORTED, "K and V must each be below 4 GiB (total_tokens %lld x %lld KV heads x head_dim %lld)",
                dims->total_tokens, dims->num_kv_heads, dims->head_dim);
  return {};
}

Error validate_segments(const br_dims& dims, const int32_t* so, const int32_t* sp) {
  if (!so || !sp) return fail(BR_ERR_INVALID_ARG, "segment_offsets and seg_ptr must be non-NULL host arrays");
  if (sp[0] != 0) return fail(BR_ERR_INVALID_ARG, "seg_ptr[0] must be 0 (got %lld)", sp[0]);
  int64_t prev_end = 0;
  for (int b = 0; b < dims.num_prompts; ++b) {
    int64_t n = int64_t(sp[b + 1]) - sp[b];
    if (n < 4)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld has %lld segment offsets; need >= 4 (instruction, >= 1 document, query)", b, n);
    const int32_t* o = so + sp[b];
    if (o[0] != prev_end)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld starts at %lld but the previous prompt ends at %lld", b, o[0], prev_end);
    if (o[1] < o[0]) return fail(BR_ERR_INVALID_ARG, "prompt %lld: instruction end %lld before its start", b, o[1]);
    for (int64_t k = 1; k < n - 1; ++k)
      if (o[k + 1] <= o[k])
        return fail(BR_ERR_INVALID_ARG, "prompt %lld: segment %lld is empty or reversed (offset %lld)", b, k, o[k + 1]);
    prev_end = o[n - 1];
    if (prev_end > dims.total_tokens)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld ends at %lld beyond total_tokens %lld", b, prev_end, dims.total_tokens);
  }
  if (prev_end != dims.total_tokens)
    return fail(BR_ERR_INVALID_ARG, "last segment offset %lld != total_tokens %lld", prev_end, dims.total_tokens);
  return {};
}

namespace {

// Shared by the prompt plan and the query-only plan.
struct ItemMaker {
  int TM, BN;
  int64_t CK;  // split-key chunk length
  int32_t tiles(int64_t a, int64_t b) const { return int32_t(b > a ? cdiv(b - a, BN) : 0); }
  AttnItem operator()(int64_t row0, int64_t lim, int64_t a0, int64_t a1, int64_t b0, int64_t b1, int32_t slot) const {
    if (a1 <= a0) a0 = a1 = 0;
    if (b1 <= b0) b0 = b1 = 0;
    return AttnItem{int32_t(row0), int32_t(lim), int32_t(a0), int32_t(a1), int32_t(b0), int32_t(b1), slot,
                    tiles(a0, a1) + tiles(b0, b1)};
  }
};

void init_plan(const br_dims& dims, int64_t max_unmasked, AttnPlan* plan, ItemMaker* mk) {
  AttnPlan& P = *plan;
  P = AttnPlan{};
  P.group = dims.num_q_heads / dims.num_kv_heads;
  P.rows_per_tile = tokens_per_tile(P.group);
  P.key_tile = kKeyTile;
  // Split-key chunk for query rows: aim for ~8 chunks of the longest unmasked key range, each
  // 4..64 key tiles, so long query tiles spread over many workgroups (measured on MI355X: 8 is
  // 2% faster than 16 for 16 prompts of 13,500 tokens, the same at 12,864 tokens; 32 and 64 are
  // slower; 100,096 tokens reach the 64-tile cap either way).
  const int64_t chunk_tiles = std::min<int64_t>(64, std::max<int64_t>(4, cdiv(cdiv(max_unmasked, kKeyTile), 8)));
  P.chunk_keys = int(chunk_tiles * kKeyTile);
  *mk = ItemMaker{P.rows_per_tile, kKeyTile, P.chunk_keys};
}

// Query rows [qs, qe): the keys of `ranges` unmasked (each range split into chunks of at most
// CK keys; partials merged afterwards when there is more than one chunk), then the query's own
// tokens [qs, row] causally (attached to the last chunk).
void add_query_rows(int64_t qs, int64_t qe, const std::vector<std::pair<int64_t, int64_t>>& ranges,
                    const ItemMaker& mk, AttnPlan* plan, std::vector<AttnItem>* out) {
  AttnPlan& P = *plan;
  std::vector<std::pair<int64_t, int64_t>> chunks;
  for (const auto& r : ranges)
    for (int64_t a = r.first; a < r.second; a += mk.CK) chunks.push_back({a, std::min(a + mk.CK, r.second)});
  for (int64_t r0 = qs; r0 < qe; r0 += mk.TM) {
    const int64_t b1 = std::min(r0 + mk.TM, qe);
    if (chunks.size() <= 1) {
      const int64_t a0 = chunks.empty() ? 0 : chunks[0].first, a1 = chunks.empty() ? 0 : chunks[0].second;
      out->push_back(mk(r0, qe, a0, a1, qs, b1, -1));
      continue;
    }
    const int32_t slot0 = P.n_slots;
    for (size_t c = 0; c < chunks.size(); ++c) {
      const bool last = c + 1 == chunks.size();
      out->push_back(mk(r0, qe, chunks[c].first, chunks[c].second, last ? qs : 0, last ? b1 : 0, slot0 + int32_t(c)));
    }
    P.merges.push_back(MergeItem{int32_t(r0), int32_t(qe), slot0, int32_t(chunks.size())});
    P.n_slots += int32_t(chunks.size());
  }
}

void add_query_rows(int64_t qs, int64_t qe, int64_t u0, int64_t u1, const ItemMaker& mk, AttnPlan* plan,
                    std::vector<AttnItem>* out) {
  std::vector<std::pair<int64_t, int64_t>> ranges;
  if (u1 > u0) ranges.push_back({u0, u1});
  add_query_rows(qs, qe, ranges, mk, plan, out);
}

Error check_item_count(const AttnPlan& plan) {
  if (int64_t(plan.items.size()) >= kMaxAttnItems)
    return fail(BR_ERR_UNSUPPORTED, "the attention plan has %lld work items; at most %lld are supported",
                (long long)plan.items.size(), kMaxAttnItems - 1);
  return {};
}

// Workspace layout (the schedule is made per device, by the caller).
void finish_plan(const br_dims& dims, AttnPlan* plan) {
  AttnPlan& P = *plan;
  const size_t hkv = size_t(dims.num_kv_heads), d = size_t(dims.head_dim);
  P.off_items = 0;
  P.off_ranges = align_up(P.items.size() * sizeof(AttnItem), 256);
  P.off_merges = align_up(P.off_ranges + size_t(kMaxAttnWgPerHead + 1) * sizeof(int32_t), 256);
  P.off_part_o = align_up(P.off_merges + P.merges.size() * sizeof(MergeItem), 256);
  P.off_part_ml = align_up(P.off_part_o + size_t(P.n_slots) * hkv * kRowsPerTile * d * 4, 256);
  P.total_bytes = align_up(P.off_part_ml + size_t(P.n_slots) * hkv * kRowsPerTile * 2 * 4, 256);
}

// Longest items first (the split query chunks), the rest after in the order given.
void order_items(std::vector<AttnItem>&& query_items, const std::vector<AttnItem>& other_items, AttnPlan* plan) {
  std::stable_sort(query_items.begin(), query_items.end(),
                   [](const AttnItem& x, const AttnItem& y) { return x.ntiles > y.ntiles; });
  plan->items = std::move(query_items);
  plan->items.insert(plan->items.end(), other_items.begin(), other_items.end());
}

}  // namespace

Error build_attn_plan(const br_dims& dims, const int32_t* so, const int32_t* sp, AttnPlan* plan) {
  Error e = validate_dims(&dims);
  if (!e.ok()) return e;
  e = validate_segments(dims, so, sp);
  if (!e.ok()) return e;

  int64_t max_prefix = 0;
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    int n = sp[b + 1] - sp[b];
    max_prefix = std::max<int64_t>(max_prefix, o[n - 2] - o[0]);
  }
  ItemMaker mk{};
  init_plan(dims, max_prefix, plan, &mk);
  const int64_t TM = mk.TM;

  std::vector<AttnItem> query_items, other_items;
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    const int n = sp[b + 1] - sp[b];
    const int64_t ps = o[0], pe = o[1], qs = o[n - 2], qe = o[n - 1];
    // instruction rows: causal within the instruction
    for (int64_t r0 = ps; r0 < pe; r0 += TM) other_items.push_back(mk(r0, pe, 0, 0, ps, std::min(r0 + TM, pe), -1));
    // document rows: whole instruction, then own document causally; last row tile first
    for (int k = 1; k <= n - 3; ++k) {
      const int64_t ds = o[k], de = o[k + 1];
      const int64_t ntile = cdiv(de - ds, TM);
      for (int64_t t = ntile - 1; t >= 0; --t) {
        const int64_t r0 = ds + t * TM;
        other_items.push_back(mk(r0, de, ps, pe, ds, std::min(r0 + TM, de), -1));
      }
    }
    // final-query rows: everything before the query unmasked, the query causally
    add_query_rows(qs, qe, ps, qs, mk, plan, &query_items);
  }
  // Time order for the list schedule: the long query chunks first, then instruction and
  // document row tiles in prompt order.  The row tiles of one document stay adjacent, so the
  // schedule hands them to different workgroups at about the same time and the document's keys
  // are fetched once and re-read from the shared L2.
  order_items(std::move(query_items), other_items, plan);
  e = check_item_count(*plan);
  if (!e.ok()) return e;
  finish_plan(dims, plan);
  return {};
}

Error validate_queries(const br_dims& dims, int32_t corpus_len, const int32_t* qo) {
  if (!qo) return fail(BR_ERR_INVALID_ARG, "query_offsets must be a non-NULL host array");
  if (corpus_len < 0) return fail(BR_ERR_INVALID_ARG, "corpus_len must be >= 0 (got %lld)", corpus_len);
  if (qo[0] != corpus_len)
    return fail(BR_ERR_INVALID_ARG, "query_offsets[0] (%lld) must equal corpus_len (%lld)", qo[0], corpus_len);
  for (int b = 0; b < dims.num_prompts; ++b)
    if (qo[b + 1] <= qo[b])
      return fail(BR_ERR_INVALID_ARG, "query %lld is empty or reversed (offsets %lld, %lld)", b, qo[b], qo[b + 1]);
  if (qo[dims.num_prompts] != dims.total_tokens)
    return fail(BR_ERR_INVALID_ARG, "last query offset %lld != total_tokens %lld", qo[dims.num_prompts], dims.total_tokens);
  return {};
}

Error build_query_plan(const br_dims& dims, int32_t corpus_len, const int32_t* qo, AttnPlan* plan) {
  Error e = validate_dims(&dims);
  if (!e.ok()) return e;
  e = validate_queries(dims, corpus_len, qo);
  if (!e.ok()) return e;
  ItemMaker mk{};
  init_plan(dims, corpus_len, plan, &mk);
  std::vector<AttnItem> query_items;
  for (int b = 0; b < dims.num_prompts; ++b) add_query_rows(qo[b], qo[b + 1], 0, corpus_len, mk, plan, &query_items);
  // Time order: corpus chunk by chunk, every query's row tiles for one chunk adjacent, so the
  // list schedule runs them at the same time and the chunk's keys are fetched once into L2.
  std::stable_sort(query_items.begin(), query_items.end(),
                   [](const AttnItem& x, const AttnItem& y) { return x.a_start < y.a_start; });
  plan->items = std::move(query_items);
  e = check_item_count(*plan);
  if (!e.ok()) return e;
  finish_plan(dims, plan);
  return {};
}

Error validate_keep(const br_dims& dims, const int32_t* so, const int32_t* sp, const int32_t* keep_ptr,
                    const int32_t* keep) {
  if (!keep_ptr || !keep) return fail(BR_ERR_INVALID_ARG, "keep_ptr and keep must be non-NULL host arrays");
  if (keep_ptr[0] != 0) return fail(BR_ERR_INVALID_ARG, "keep_ptr[0] must be 0 (got %lld)", keep_ptr[0]);
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int64_t n_docs = int64_t(sp[b + 1]) - sp[b] - 3;
    const int64_t k0 = keep_ptr[b], k1 = keep_ptr[b + 1];
    if (k1 < k0) return fail(BR_ERR_INVALID_ARG, "keep_ptr decreases at prompt %lld", b);
    std::vector<char> seen(size_t(n_docs), 0);
    for (int64_t k = k0; k < k1; ++k) {
      const int32_t doc = keep[k];
      if (doc < 0 || doc >= n_docs)
        return fail(BR_ERR_INVALID_ARG, "prompt %lld: kept document %lld out of range [0, %lld)", b, doc, n_docs);
      if (seen[size_t(doc)]) return fail(BR_ERR_INVALID_ARG, "prompt %lld: document %lld kept twice", b, doc);
      seen[size_t(doc)] = 1;
    }
  }
  return {};
}

Error build_routed_plan(const br_dims& dims, const int32_t* so, const int32_t* sp, const int32_t* keep_ptr,
                        const int32_t* keep, AttnPlan* plan) {
  Error e = validate_dims(&dims);
  if (!e.ok()) return e;
  e = validate_segments(dims, so, sp);
  if (!e.ok()) return e;
  e = validate_keep(dims, so, sp, keep_ptr, keep);
  if (!e.ok()) return e;

  // Per prompt: the unmasked key ranges of the query rows (instruction plus kept documents, runs
  // of adjacent spans merged) and their longest total, which sizes the chunks.
  std::vector<std::vector<std::pair<int64_t, int64_t>>> qranges(size_t(dims.num_prompts));
  std::vector<std::vector<char>> kept(size_t(dims.num_prompts));
  int64_t max_unmasked = 0;
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    const int n = sp[b + 1] - sp[b];
    kept[size_t(b)].assign(size_t(n - 3), 0);
    for (int64_t k = keep_ptr[b]; k < keep_ptr[b + 1]; ++k) kept[size_t(b)][size_t(keep[k])] = 1;
    auto& rs = qranges[size_t(b)];
    auto add = [&](int64_t a, int64_t z) {
      if (z <= a) return;
      if (!rs.empty() && rs.back().second == a)
        rs.back().second = z;
      else
        rs.push_back({a, z});
    };
    add(o[0], o[1]);
    for (int k = 1; k <= n - 3; ++k)
      if (kept[size_t(b)][size_t(k - 1)]) add(o[k], o[k + 1]);
    int64_t tot = 0;
    for (const auto& r : rs) tot += r.second - r.first;
    max_unmasked = std::max(max_unmasked, tot);
  }
  ItemMaker mk{};
  init_plan(dims, max_unmasked, plan, &mk);
  const int64_t TM = mk.TM;
  std::vector<AttnItem> query_items, other_items;
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    const int n = sp[b + 1] - sp[b];
    const int64_t ps = o[0], pe = o[1], qs = o[n - 2], qe = o[n - 1];
    for (int64_t r0 = ps; r0 < pe; r0 += TM) other_items.push_back(mk(r0, pe, 0, 0, ps, std::min(r0 + TM, pe), -1));
    for (int k = 1; k <= n - 3; ++k) {
      if (!kept[size_t(b)][size_t(k - 1)]) continue;  // dropped documents' rows are not computed
      const int64_t ds = o[k], de = o[k + 1];
      const int64_t ntile = cdiv(de - ds, TM);
      for (int64_t t = ntile - 1; t >= 0; --t) {
        const int64_t r0 = ds + t * TM;
        other_items.push_back(mk(r0, de, ps, pe, ds, std::min(r0 + TM, de), -1));
      }
    }
    add_query_rows(qs, qe, qranges[size_t(b)], mk, plan, &query_items);
  }
  order_items(std::move(query_items), other_items, plan);
  e = check_item_count(*plan);
  if (!e.ok()) return e;
  finish_plan(dims, plan);
  return {};
}

int64_t attn_item_cost(const AttnItem& it) {
  // Measured on gfx950: a key tile of a split query chunk (keys streamed from memory, fp32
  // partials) costs about 1.25 document key tiles; loading a row tile's queries and storing its
  // outputs about two key tiles (the kernel overlaps them with the neighbouring items' tiles).
  // Against per-item costs of 1, 4 and 8 key tiles (same split-chunk slope): 2 was fastest or
  // within noise at the worked, long, batched and ragged shapes (worked -4%, batched -1% from 4).
  return it.slot < 0 ? 4 * int64_t(it.ntiles) + 8 : 5 * int64_t(it.ntiles) + 16;
}

void schedule_attn_plan(int num_kv_heads, int workgroups, AttnPlan* plan) {
  AttnPlan& P = *plan;
  // Greedy list schedule: walk the items in time order and give each to the workgroup of the KV
  // head that becomes free first (ties to the lowest index), as a shared work queue would at run
  // time, but fixed in advance so the kernel needs no atomics.  Workgroups that run at the same
  // time therefore work on neighbouring items, and the largest imbalance is one item's cost.
  const int64_t n_items = int64_t(P.items.size());
  const int W = int(std::max<int64_t>(1, std::min<int64_t>({n_items, int64_t(std::max(1, workgroups)) / num_kv_heads,
                                                             int64_t(kMaxAttnWgPerHead)})));
  P.wg_per_head = W;
  std::vector<int32_t> owner(static_cast<size_t>(n_items));
  std::vector<int32_t> count(size_t(W), 0);
  std::vector<int64_t> free_at(size_t(W), 0);  // time each workgroup becomes free
  for (int64_t i = 0; i < n_items; ++i) {
    // earliest-free workgroup, ties to the lowest index (a linear scan over at most a few
    // hundred workgroups is cheaper than a heap here)
    int best = 0;
    int64_t t = free_at[0];
    for (int w = 1; w < W; ++w)
      if (free_at[size_t(w)] < t) {
        t = free_at[size_t(w)];
        best = w;
      }
    owner[size_t(i)] = best;
    ++count[size_t(best)];
    free_at[size_t(best)] = t + attn_item_cost(P.items[size_t(i)]);
  }
  P.ranges.assign(size_t(W) + 1, 0);
  for (int w = 0; w < W; ++w) P.ranges[size_t(w) + 1] = P.ranges[size_t(w)] + count[size_t(w)];
  std::vector<int32_t> fill(P.ranges.begin(), P.ranges.end() - 1);
  P.sched.resize(size_t(n_items));
  for (int64_t i = 0; i < n_items; ++i) P.sched[size_t(fill[size_t(owner[size_t(i)])]++)] = P.items[size_t(i)];
}

Error validate_docs(const br_dims& dims, int32_t n_signal, const int32_t* dof, const int32_t* dp) {
  Error e = validate_dims(&dims);
  if (!e.ok()) return e;
  if (!dof || !dp) return fail(BR_ERR_INVALID_ARG, "doc_offsets and doc_ptr must be non-NULL host arrays");
  if (n_signal < 1) return fail(BR_ERR_INVALID_ARG, "n_signal must be >= 1 (got %lld)", n_signal);
  if (n_signal > 64) return fail(BR_ERR_UNSUPPORTED, "n_signal %lld exceeds 64", n_signal);
  if (int64_t(n_signal) * dims.num_q_heads > 4096)
    return fail(BR_ERR_UNSUPPORTED, "n_signal * num_q_heads = %lld exceeds 4096", int64_t(n_signal) * dims.num_q_heads);
  if (dp[0] != 0) return fail(BR_ERR_INVALID_ARG, "doc_ptr[0] must be 0 (got %lld)", dp[0]);
  for (int b = 0; b < dims.num_prompts; ++b) {
    int64_t n = int64_t(dp[b + 1]) - dp[b];
    if (n < 2) return fail(BR_ERR_INVALID_ARG, "prompt %lld has %lld document offsets; need >= 2", b, n);
    const int32_t* o = dof + dp[b];
    if (o[0] < 0) return fail(BR_ERR_INVALID_ARG, "prompt %lld: document offset %lld is negative", b, o[0]);
    for (int64_t k = 0; k + 1 < n; ++k)
      if (o[k + 1] <= o[k])
        return fail(BR_ERR_INVALID_ARG, "prompt %lld: document %lld is empty or reversed (offset %lld)", b, k, o[k + 1]);
    if (o[n - 1] > dims.total_tokens)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld: documents end at %lld beyond total_tokens %lld", b, o[n - 1],
                  dims.total_tokens);
  }
  return {};
}

Error build_score_plan(const br_dims& dims, int32_t n_signal, const int32_t* dof, const int32_t* dp, ScorePlan* plan) {
  Error e = validate_docs(dims, n_signal, dof, dp);
  if (!e.ok()) return e;
  ScorePlan& P = *plan;
  P = ScorePlan{};
  P.group = dims.num_q_heads / dims.num_kv_heads;
  P.n_signal = n_signal;
  P.rows_per_kv = n_signal * P.group;
  P.row_blocks = int(cdiv(P.rows_per_kv, kRowsPerWave));
  const int B = dims.num_prompts;
  int64_t doc_tokens = 0;
  P.prompt_score_base.resize(B + 1);
  for (int b = 0; b <= B; ++b) P.prompt_score_base[b] = dp[b] - b;
  P.n_docs = P.prompt_score_base[B];
  for (int b = 0; b < B; ++b) doc_tokens += dof[dp[b + 1] - 1] - dof[dp[b]];
  // About 4096 waves in total; each wave streams whole documents.
  const int64_t waves_per_item = int64_t(dims.num_kv_heads) * P.row_blocks;
  const int64_t want_items = std::max<int64_t>(1, 4096 / waves_per_item);
  const int64_t target = std::max<int64_t>(32, cdiv(doc_tokens, want_items));
  for (int b = 0; b < B; ++b) {
    int32_t d0 = dp[b];
    const int32_t dend = dp[b + 1] - 1;  // global index one past the last document of prompt b
    while (d0 < dend) {
      int32_t d1 = d0 + 1;
      while (d1 < dend && dof[d1] - dof[d0] < target) ++d1;
      P.items.push_back(ScoreItem{b, d0, d1, P.prompt_score_base[b] + (d0 - dp[b])});
      d0 = d1;
    }
  }
  const size_t n_off = size_t(dp[B]);
  P.off_items = 0;
  P.off_doc_offsets = align_up(P.items.size() * sizeof(ScoreItem), 256);
  P.off_prompt_base = align_up(P.off_doc_offsets + n_off * 4, 256);
  P.off_ml = align_up(P.off_prompt_base + size_t(B + 1) * 4, 256);
  // [n_docs, RT] per-document (max, sum) partials followed by [B, RT] per-row (max, 1/Z)
  const size_t rt = size_t(n_signal) * size_t(dims.num_q_heads);
  P.total_bytes = align_up(P.off_ml + (size_t(P.n_docs) + size_t(B)) * rt * 8, 256);
  return {};
}

}  // namespace br
