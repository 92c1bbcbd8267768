// Host-side plans outside the forward attention: rotary-embedding position runs, the backward's
// key-major items and workspace layout, the readout backward's layout and InfoNCE validation.
// Pure C++ (no HIP calls), unit-testable without a GPU.
#include <algorithm>
#include <limits>
#include <climits>
#include <cmath>
#include <cstdio>
#include <vector>

#include "plan.h"

namespace br {
namespace {

Error fail(br_status s, const char* fmt, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b, c);
  return Error{s, buf};
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// rotary embedding runs

size_t rope_workspace_bytes(int64_t n_runs, int head_dim) {
  return align_up(size_t(n_runs + 1) * 4, 16) + align_up(size_t(n_runs) * 4, 16) + size_t(head_dim / 2) * 8;
}

Error validate_rope(const br_dims& dims, float rope_theta, int32_t query_pos0) {
  if (!(rope_theta > 0.f) || std::isinf(rope_theta))
    return Error{BR_ERR_INVALID_ARG, "rope_theta must be finite and positive"};
  if (query_pos0 < 0) return fail(BR_ERR_INVALID_ARG, "query_pos0 must be >= 0 (got %lld)", query_pos0);
  (void)dims;
  return {};
}

namespace {

void finish_rope(const br_dims& dims, float theta, RopePlan* plan) {
  const int half = dims.head_dim / 2;
  plan->inv_freq.resize(size_t(half));
  for (int k = 0; k < half; ++k) plan->inv_freq[size_t(k)] = std::pow(double(theta), -2.0 * k / dims.head_dim);
  const int64_t n = int64_t(plan->pos0.size());
  plan->off_start = 0;
  plan->off_pos0 = align_up(size_t(n + 1) * 4, 16);
  plan->off_freq = plan->off_pos0 + align_up(size_t(n) * 4, 16);
  plan->total_bytes = plan->off_freq + size_t(half) * 8;
}

}  // namespace

Error build_rope_plan(const br_dims& dims, const int32_t* so, const int32_t* sp, float rope_theta, int32_t query_pos0,
                      int32_t docs_after_instruction, RopePlan* plan) {
  Error e = validate_segments(dims, so, sp);
  if (!e.ok()) return e;
  e = validate_rope(dims, rope_theta, query_pos0);
  if (!e.ok()) return e;
  *plan = RopePlan{};
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    const int64_t n = int64_t(sp[b + 1]) - sp[b];
    const int32_t p = o[1] - o[0];
    if (int64_t(query_pos0) + (o[n - 1] - o[n - 2]) > INT32_MAX)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld: query positions from %lld overflow int32", b, query_pos0);
    auto add = [&](int32_t start, int32_t end, int32_t pos0) {
      if (end <= start) return;
      plan->start.push_back(start);
      plan->pos0.push_back(pos0);
    };
    add(o[0], o[1], 0);
    for (int64_t k = 1; k < n - 2; ++k) add(o[k], o[k + 1], docs_after_instruction ? p : 0);
    add(o[n - 2], o[n - 1], query_pos0);
  }
  plan->rows = dims.total_tokens;
  plan->start.push_back(int32_t(dims.total_tokens));
  finish_rope(dims, rope_theta, plan);
  return {};
}

Error build_rope_signal_plan(const br_dims& dims, int32_t n_signal, const int32_t* so, const int32_t* sp,
                             float rope_theta, int32_t query_pos0, RopePlan* plan) {
  Error e = validate_segments(dims, so, sp);
  if (!e.ok()) return e;
  e = validate_rope(dims, rope_theta, query_pos0);
  if (!e.ok()) return e;
  if (n_signal < 1) return fail(BR_ERR_INVALID_ARG, "n_signal must be >= 1 (got %lld)", n_signal);
  *plan = RopePlan{};
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    const int64_t n = int64_t(sp[b + 1]) - sp[b];
    const int64_t q = o[n - 1] - o[n - 2];
    if (q < n_signal)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld: query has %lld tokens, fewer than n_signal = %lld", b, q, n_signal);
    if (int64_t(query_pos0) + q > INT32_MAX)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld: query positions from %lld overflow int32", b, query_pos0);
    plan->start.push_back(int32_t(int64_t(b) * n_signal));
    plan->pos0.push_back(int32_t(query_pos0 + q - n_signal));
  }
  plan->rows = int64_t(dims.num_prompts) * n_signal;
  plan->start.push_back(int32_t(plan->rows));
  finish_rope(dims, rope_theta, plan);
  return {};
}

// ---------------------------------------------------------------------------------------------
// backward plan

Error build_bwd_plan(const br_dims& dims, const int32_t* so, const int32_t* sp, BwdPlan* plan) {
  *plan = BwdPlan{};
  Error e = build_attn_plan(dims, so, sp, &plan->fwd);
  if (!e.ok()) return e;
  BwdPlan& P = *plan;
  // Order key of each item: split items -1 (first), a prompt's instruction keys 0, document keys
  // their group (1, 2, ...), query keys last.
  std::vector<int64_t> order_key;
  int64_t cur_key = 0;
  auto add_keys = [&](int64_t ks, int64_t ke, int64_t u0, int64_t u1) {
    for (int64_t k0 = ks; k0 < ke; k0 += kBwdKeyTile) {
      const int64_t kl = std::min<int64_t>(k0 + kBwdKeyTile, ke);
      const int64_t nu = u1 > u0 ? u1 - u0 : 0;
      if (nu <= kBwdRowChunk) {
        P.kv_items.push_back(KvItem{int32_t(k0), int32_t(kl), int32_t(k0), int32_t(ke), int32_t(nu ? u0 : 0),
                                    int32_t(nu ? u1 : 0), -1, int32_t(ke - k0 + nu)});
        order_key.push_back(cur_key);
        continue;
      }
      const int32_t slot0 = P.kv_slots;
      int32_t n = 0;
      for (int64_t a = u0; a < u1; a += kBwdRowChunk, ++n) {
        const int64_t b = std::min<int64_t>(a + kBwdRowChunk, u1);
        const bool first = a == u0;  // the first chunk also takes the causal rows
        P.kv_items.push_back(KvItem{int32_t(k0), int32_t(kl), int32_t(first ? k0 : 0), int32_t(first ? ke : 0),
                                    int32_t(a), int32_t(b), slot0 + n, int32_t((first ? ke - k0 : 0) + (b - a))});
        order_key.push_back(-1);
      }
      P.kv_merges.push_back(KvMerge{int32_t(k0), int32_t(kl), slot0, n});
      P.kv_slots += n;
    }
  };
  int64_t group = 1, group_tokens = 0;
  for (int b = 0; b < dims.num_prompts; ++b) {
    const int32_t* o = so + sp[b];
    const int n = sp[b + 1] - sp[b];
    const int64_t ps = o[0], pe = o[1], qs = o[n - 2], qe = o[n - 1];
    cur_key = 0;
    add_keys(ps, pe, pe, qe);  // instruction keys: every later row
    for (int k = 1; k <= n - 3; ++k) {  // document keys: the document causally, then the query
      if (group_tokens >= kBwdGroupTokens) {
        ++group;
        group_tokens = 0;
      }
      cur_key = group;
      group_tokens += o[k + 1] - o[k];
      add_keys(o[k], o[k + 1], qs, qe);
    }
    cur_key = std::numeric_limits<int64_t>::max();
    add_keys(qs, qe, 0, 0);  // query keys: the query, causally
  }
  // Launch order: the split instruction chunks first (the longest items, so they start early),
  // then the instruction keys of short prompts, then the documents group by group, the query keys
  // last; longest first inside each class and group.  A group's key tiles run close together, so
  // the rows that several of them read come from the L2 (measured at the long prompt: 2.43 ->
  // 2.35 ms for the whole backward against a single longest-first order, and 4.75 -> 4.57 ms for
  // the 16-prompt batch; groups of 4 to 16 documents of 200 tokens did equally well, a document's
  // tiles alone were slower).
  {
    std::vector<size_t> idx(P.kv_items.size());
    for (size_t i = 0; i < idx.size(); ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(), [&](size_t x, size_t y) {
      if (order_key[x] != order_key[y]) return order_key[x] < order_key[y];
      return P.kv_items[x].rows > P.kv_items[y].rows;
    });
    std::vector<KvItem> sorted;
    sorted.reserve(idx.size());
    for (size_t i : idx) sorted.push_back(P.kv_items[i]);
    P.kv_items.swap(sorted);
  }
  const size_t hkv = size_t(dims.num_kv_heads), hq = size_t(dims.num_q_heads), d = size_t(dims.head_dim);
  P.off_items = 0;
  P.off_merges = align_up(P.fwd.items.size() * sizeof(AttnItem), 256);
  P.off_kv_items = align_up(P.off_merges + P.fwd.merges.size() * sizeof(MergeItem), 256);
  P.off_kv_merges = align_up(P.off_kv_items + P.kv_items.size() * sizeof(KvItem), 256);
  P.off_part_dq = align_up(P.off_kv_merges + P.kv_merges.size() * sizeof(KvMerge), 256);
  P.off_part_dkv = align_up(P.off_part_dq + size_t(P.fwd.n_slots) * hkv * kRowsPerTile * d * 4, 256);
  P.off_dvec = align_up(P.off_part_dkv + size_t(P.kv_slots) * hkv * kBwdKeyTile * d * 4 * 2, 256);
  P.total_bytes = align_up(P.off_dvec + size_t(dims.total_tokens) * hq * 4 * 2, 256);  // Dr, then -lse log2(e)
  return {};
}

// ---------------------------------------------------------------------------------------------
// readout backward and InfoNCE

Error build_doc_bwd_plan(const br_dims& dims, int32_t n_signal, const int32_t* dof, const int32_t* dp,
                         DocBwdPlan* plan) {
  *plan = DocBwdPlan{};
  Error e = build_score_plan(dims, n_signal, dof, dp, &plan->fwd);
  if (!e.ok()) return e;
  DocBwdPlan& P = *plan;
  if (P.fwd.rows_per_kv > kDocBwdMaxRows)
    return fail(BR_ERR_UNSUPPORTED, "readout backward supports n_signal * G <= %lld signal rows per KV head (got %lld)",
                kDocBwdMaxRows, P.fwd.rows_per_kv);
  const int B = dims.num_prompts;
  P.prompt_items.assign(size_t(B) + 1, 0);
  for (const ScoreItem& it : P.fwd.items) P.prompt_items[size_t(it.prompt) + 1]++;
  for (int b = 0; b < B; ++b) P.prompt_items[size_t(b) + 1] += P.prompt_items[size_t(b)];
  const size_t rt = size_t(n_signal) * size_t(dims.num_q_heads);
  const size_t rb = size_t(P.fwd.row_blocks);
  P.off_prompt_items = align_up(P.fwd.total_bytes, 256);
  P.off_center = align_up(P.off_prompt_items + size_t(B + 1) * 4, 256);
  P.off_part = align_up(P.off_center + size_t(B) * rt * 4, 256);
  P.total_bytes = align_up(P.off_part + P.fwd.items.size() * size_t(dims.num_kv_heads) * rb * kRowsPerWave *
                                            size_t(dims.head_dim) * 4, 256);
  return {};
}

size_t infonce_workspace_bytes(int32_t num_prompts) {
  return align_up(size_t(num_prompts + 1) * 4, 256) + align_up(size_t(num_prompts) * 4, 256);
}

Error validate_infonce(int32_t num_prompts, const int32_t* dp, const int32_t* gold, float tau) {
  if (num_prompts < 1) return fail(BR_ERR_INVALID_ARG, "num_prompts must be >= 1 (got %lld)", num_prompts);
  if (!dp || !gold) return fail(BR_ERR_INVALID_ARG, "doc_ptr and gold must be non-NULL host arrays");
  if (!(tau > 0.f) || std::isinf(tau)) return Error{BR_ERR_INVALID_ARG, "tau must be finite and positive"};
  if (dp[0] != 0) return fail(BR_ERR_INVALID_ARG, "doc_ptr[0] must be 0 (got %lld)", dp[0]);
  for (int b = 0; b < num_prompts; ++b) {
    const int64_t n = int64_t(dp[b + 1]) - dp[b] - 1;
    if (n < 1) return fail(BR_ERR_INVALID_ARG, "prompt %lld has no documents", b);
    if (n > kInfoNceMaxDocs)
      return fail(BR_ERR_UNSUPPORTED, "prompt %lld has %lld documents; at most %lld", b, n, kInfoNceMaxDocs);
    if (gold[b] < 0 || gold[b] >= n)
      return fail(BR_ERR_INVALID_ARG, "prompt %lld: gold index %lld outside [0, %lld)", b, gold[b], n);
  }
  return {};
}

}  // namespace br
