// Attention-mass document scores on gfx950 (BlockRank summary, "Score computation procedure"
// steps 1-4; blog, attention supervision):
//   z_{ihj}      = Q_S[i,h] . K[j, h/G] * scale          for j in the prompt's document tokens
//   alpha'_{ihj} = softmax over all document tokens j of z_{ihj}
//   s_k          = (1/Hq) sum_h sum_i sum_{j in d_k} alpha'_{ihj}
//
// Three kernels, all streaming each document key once from HBM:
//   1. doc_partial_kernel: one wave per (document group, KV head, 32-row block).  The wave's
//      rows are (signal token, query head) pairs of one KV group; logits come from the
//      32x32x16 bf16 MFMA with keys on M.  For every document it keeps a running (max, sum of
//      exp2) per row and writes (m_k, e_k) at the document's end (a segmented reduction over
//      document spans; key tiles start at each document's first token).
//   2. doc_rowstat_kernel: per row, M = max_k m_k and Z = sum_k e_k 2^(m_k - M).
//   3. doc_final_kernel: one workgroup per document, head_scores[h,k] = sum_i e_k 2^(m_k - M)/Z
//      and s_k = mean over heads, summed in a fixed order (deterministic).
#include "attn_merge.h"
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace br {

template <int D>
__device__ __forceinline__ void doc_partial_block(int64_t block, const uint16_t* __restrict__ Q_S,
                                                  const uint16_t* __restrict__ K, const ScoreItem* __restrict__ items,
                                                  const int32_t* __restrict__ dof, float2* __restrict__ ml,
                                                  int64_t n_items, int Hq, int Hkv, int n_signal, int row_blocks,
                                                  float scale_log2) {
  constexpr int DSTEPS = D / 16;
  const int lane = threadIdx.x & 63, n = lane & 31, half = lane >> 5;
  const int64_t wid = block * 4 + (threadIdx.x >> 6);
  if (wid >= n_items * Hkv * row_blocks) return;  // whole wave exits together
  const int g = int(wid % Hkv);
  const int64_t rest = wid / Hkv;
  const int rb = int(rest % row_blocks);
  const ScoreItem it = items[rest / row_blocks];
  const int G = Hq / Hkv;
  const int rho = rb * 32 + n;
  const bool row_ok = rho < n_signal * G;
  const int i = rho / G, h = g * G + rho % G;
  const int RT = n_signal * Hq;
  const int64_t kv_stride = int64_t(Hkv) * D;

  // Head-dim order inside the MFMA contraction: at step st lane half `half` supplies elements
  // 16*st + 8*half .. +8 (any order works if Q and K agree).
  u32x4_t qf[DSTEPS];
  {
    const uint16_t* qp = Q_S + ((int64_t(it.prompt) * n_signal + i) * Hq + h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) qf[s] = row_ok ? load16(qp + 16 * s) : u32x4_t{0, 0, 0, 0};
  }
  // Keys move as whole rows: instruction s of a step reads KRI key rows (1 KB, 8 full cache
  // lines; lane l takes 16-byte chunk l % KCH of row KRI s + l / KCH) instead of 32 B from each
  // of 32 rows.  Each wave passes its 32 rows through its own LDS region [key][D + 8] into MFMA
  // fragments; a wave's LDS operations complete in order, so no barrier is needed.
  constexpr int KCH = D / 8, KRI = 512 / D, KROW = D + 8;
  static_assert(KRI * DSTEPS == 32, "one key row block per step");
  __shared__ __align__(16) uint16_t kst_all[4][32 * KROW];
  uint16_t* const kst = kst_all[threadIdx.x >> 6];
  const uint16_t* const kbase = K + int64_t(g) * D;
  auto load_rows = [&](int t0, int end, u32x4_t* kr) {
    const rsrc_t r = make_rsrc(kbase + int64_t(t0) * kv_stride, max(0, min(32, end - t0)) * int(kv_stride) * 2);
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s)
      kr[s] = buf_load16(r, uint32_t(((KRI * s + lane / KCH) * kv_stride + 8 * (lane % KCH)) * 2));
  };
  // One register set of raw rows: they go to LDS before the next block's loads reuse them, so
  // the wave holds raw rows, fragments and Q (about 112 registers) and four waves share a SIMD.
  auto stage = [&](const u32x4_t* kr) {
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s)
      *reinterpret_cast<u32x4_t*>(&kst[(KRI * s + lane / KCH) * KROW + 8 * (lane % KCH)]) = kr[s];
  };
  auto read_frags = [&](u32x4_t* kf) {
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) kf[s] = load16(&kst[n * KROW + 16 * s + 8 * half]);
  };

  int d = it.d0;
  int a = dof[d], e = dof[d + 1];
  int t0 = a;
  u32x4_t kraw[DSTEPS], kf[DSTEPS];
  load_rows(t0, e, kraw);
  float m_run = -INFINITY, e_run = 0.f;
  while (true) {
    stage(kraw);
    int nd = d, nt0 = t0 + 32, ne = e;
    if (nt0 >= e) {
      nd = d + 1;
      if (nd < it.d1) { nt0 = dof[nd]; ne = dof[nd + 1]; }
    }
    const bool has_next = nd < it.d1;
    if (has_next) load_rows(nt0, ne, kraw);
    read_frags(kf);

    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int st = 0; st < DSTEPS; ++st) s = mfma32(kf[st], qf[st], s);
    if (t0 + 32 > e) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = t0 + 8 * (r >> 2) + 4 * half + (r & 3);
        s[r] = j < e ? s[r] : -INFINITY;
      }
    }
    float mt = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
    const float m_new = fmaxf(m_run, mt * scale_log2);
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc += fast_exp2(fmaf(s[r], scale_log2, -mu));
    e_run = fmaf(e_run, fast_exp2(m_run - mu), acc);  // explicit: the body is inlined into two kernels
    m_run = m_new;

    if (t0 + 32 >= e) {  // document d is complete: combine the two halves and store (m_k, e_k)
      const float mo = other_half(m_run), eo = other_half(e_run);
      const float M = fmaxf(m_run, mo);
      const float E = fmaf(e_run, fast_exp2(m_run - M), eo * fast_exp2(mo - M));
      if (row_ok && half == 0) ml[int64_t(it.score_base + (d - it.d0)) * RT + int64_t(i) * Hq + h] = float2{M, E};
      m_run = -INFINITY;
      e_run = 0.f;
    }
    if (!has_next) break;
    d = nd; t0 = nt0; e = ne;
  }
}

template <int D>
__global__ __launch_bounds__(256, 4) void doc_partial_kernel(const uint16_t* __restrict__ Q_S,
                                                          const uint16_t* __restrict__ K,
                                                          const ScoreItem* __restrict__ items,
                                                          const int32_t* __restrict__ dof, float2* __restrict__ ml,
                                                          int64_t n_items, int Hq, int Hkv, int n_signal,
                                                          int row_blocks, float scale_log2) {
  doc_partial_block<D>(blockIdx.x, Q_S, K, items, dof, ml, n_items, Hq, Hkv, n_signal, row_blocks, scale_log2);
}

// The attention's split-key merge (workgroups [0, merge_blocks)) and the readout's partials (the
// rest) in one launch: both only read what earlier launches wrote, and neither reads the other's
// output.
template <int D>
__global__ __launch_bounds__(256, 4) void merge_doc_partial_kernel(
    int merge_blocks, uint16_t* __restrict__ O, float* __restrict__ lse, const MergeItem* __restrict__ merges,
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int G, int q_row_base, float sink_log2,
    const uint16_t* __restrict__ Q_S, const uint16_t* __restrict__ K, const ScoreItem* __restrict__ items,
    const int32_t* __restrict__ dof, float2* __restrict__ ml, int64_t n_items, int Hq, int Hkv, int n_signal,
    int row_blocks, float scale_log2) {
  if (int(blockIdx.x) < merge_blocks)
    attn_merge_block<D>(blockIdx.x, O, lse, merges, part_o, part_ml, Hq, Hkv, G, q_row_base, sink_log2);
  else
    doc_partial_block<D>(int64_t(blockIdx.x) - merge_blocks, Q_S, K, items, dof, ml, n_items, Hq, Hkv, n_signal,
                         row_blocks, scale_log2);
}

// rowstat[b * RT + r] = (M, 1/Z) for row r = i*Hq + h of prompt b, with M = max_k m_k and
// Z = sum_k e_k 2^(m_k - M).  A workgroup covers 4 rows x 64 document lanes; each lane keeps an
// online (max, sum) over its documents, and the 64 lanes of a row are combined in a fixed order.
constexpr int kStatRows = 4;
constexpr int kStatLanes = 64;
__global__ __launch_bounds__(256) void doc_rowstat_kernel(const float2* __restrict__ ml,
                                                          const int32_t* __restrict__ prompt_base,
                                                          float2* __restrict__ rowstat, int RT, int row_groups) {
  __shared__ float2 red[kStatRows][kStatLanes];
  const int b = blockIdx.x / row_groups, rg = blockIdx.x % row_groups;
  const int rl = threadIdx.x % kStatRows, kl = threadIdx.x / kStatRows;
  const int r = rg * kStatRows + rl;
  const int k0 = prompt_base[b], k1 = prompt_base[b + 1];
  float M = -INFINITY, Z = 0.f;
  if (r < RT)
    for (int k = k0 + kl; k < k1; k += kStatLanes) {
      const float2 v = ml[int64_t(k) * RT + r];
      const float Mn = fmaxf(M, v.x);
      Z = Z * fast_exp2(M - Mn) + v.y * fast_exp2(v.x - Mn);
      M = Mn;
    }
  red[rl][kl] = float2{M, Z};
  __syncthreads();
  if (kl == 0 && r < RT) {
    float Mt = -INFINITY;
    for (int t = 0; t < kStatLanes; ++t) Mt = fmaxf(Mt, red[rl][t].x);
    float Zt = 0.f;
    for (int t = 0; t < kStatLanes; ++t) Zt += red[rl][t].y * fast_exp2(red[rl][t].x - Mt);
    rowstat[int64_t(b) * RT + r] = float2{Mt, 1.f / Zt};
  }
}

// One workgroup per document k: every (signal row, head) pair contributes e_k 2^(m_k - M) / Z;
// head_scores[h,k] sums them over signal rows and s_k averages over heads, both in a fixed order.
__global__ __launch_bounds__(256) void doc_final_kernel(const float2* __restrict__ ml,
                                                        const float2* __restrict__ rowstat,
                                                        const int32_t* __restrict__ prompt_base,
                                                        float* __restrict__ scores, float* __restrict__ head_scores,
                                                        int num_prompts, int n_signal, int Hq, int n_docs) {
  __shared__ float contrib[4096];
  __shared__ float hsum[4096];
  const int k = blockIdx.x;
  int lo = 0, hi = num_prompts;  // prompt b with prompt_base[b] <= k < prompt_base[b+1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prompt_base[mid] <= k) lo = mid; else hi = mid;
  }
  const int RT = n_signal * Hq;
  const float2* mk = ml + int64_t(k) * RT;
  const float2* rs = rowstat + int64_t(lo) * RT;
  for (int r = threadIdx.x; r < RT; r += blockDim.x) {
    const float2 v = mk[r], st = rs[r];
    contrib[r] = v.y * fast_exp2(v.x - st.x) * st.y;
  }
  __syncthreads();
  for (int h = threadIdx.x; h < Hq; h += blockDim.x) {
    float hs = 0.f;
    for (int i = 0; i < n_signal; ++i) hs += contrib[i * Hq + h];
    hsum[h] = hs;
    if (head_scores) head_scores[int64_t(h) * n_docs + k] = hs;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float total = 0.f;
    for (int h = 0; h < Hq; ++h) total += hsum[h];
    scores[k] = total / float(Hq);
  }
}

// Workgroups of the readout's partial kernel (four waves each).
static int64_t doc_partial_blocks(const ScoreLaunch& a) {
  return (a.n_items * a.num_kv_heads * a.row_blocks + 3) / 4;
}

template <int D>
static hipError_t launch_merge_doc_partial_t(const AttnLaunch* m, const ScoreLaunch& a, hipStream_t stream) {
  const int merge_blocks = m ? int(m->n_merges * m->num_kv_heads * merge_wg_per_tile<D>()) : 0;
  const dim3 grid(unsigned(merge_blocks + doc_partial_blocks(a)));
  if (merge_blocks == 0) {
    doc_partial_kernel<D><<<grid, 256, 0, stream>>>(a.Q_S, a.K, a.items, a.doc_offsets, a.ml, a.n_items, a.num_q_heads,
                                                    a.num_kv_heads, a.n_signal, a.row_blocks, a.scale_log2);
  } else {
    merge_doc_partial_kernel<D><<<grid, 256, 0, stream>>>(
        merge_blocks, m->O, m->lse, m->merges, m->part_o, m->part_ml, m->num_q_heads / m->num_kv_heads,
        m->q_row_base, m->sink_log2, a.Q_S, a.K, a.items, a.doc_offsets, a.ml, a.n_items, a.num_q_heads, a.num_kv_heads,
        a.n_signal, a.row_blocks, a.scale_log2);
  }
  return hipGetLastError();
}

// The readout's partials (with the attention's deferred merge when `m` is given), then its row
// statistics.
static hipError_t launch_stats(const AttnLaunch* m, const ScoreLaunch& a, hipStream_t stream) {
  if (m && (m->head_dim != a.head_dim || m->num_q_heads != a.num_q_heads || m->num_kv_heads != a.num_kv_heads))
    return hipErrorInvalidValue;
  hipError_t e;
  if (a.head_dim == 128)
    e = launch_merge_doc_partial_t<128>(m, a, stream);
  else if (a.head_dim == 64)
    e = launch_merge_doc_partial_t<64>(m, a, stream);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const int RT = a.n_signal * a.num_q_heads;
  const int row_groups = (RT + kStatRows - 1) / kStatRows;
  float2* rowstat = a.ml + int64_t(a.n_docs) * RT;
  doc_rowstat_kernel<<<dim3(unsigned(a.num_prompts * row_groups)), 256, 0, stream>>>(a.ml, a.prompt_base, rowstat,
                                                                                      RT, row_groups);
  return hipGetLastError();
}

hipError_t launch_doc_stats(const ScoreLaunch& a, hipStream_t stream) { return launch_stats(nullptr, a, stream); }

static hipError_t launch_final(const ScoreLaunch& a, hipStream_t stream) {
  const int RT = a.n_signal * a.num_q_heads;
  const float2* rowstat = a.ml + int64_t(a.n_docs) * RT;
  doc_final_kernel<<<dim3(unsigned(a.n_docs)), 256, 0, stream>>>(
      a.ml, rowstat, a.prompt_base, a.scores, a.head_scores, a.num_prompts, a.n_signal, a.num_q_heads, a.n_docs);
  return hipGetLastError();
}

hipError_t launch_merge_doc_scores(const AttnLaunch& attn, const ScoreLaunch& a, hipStream_t stream) {
  hipError_t e = launch_stats(&attn, a, stream);
  if (e != hipSuccess) return e;
  return launch_final(a, stream);
}

hipError_t launch_doc_scores(const ScoreLaunch& a, hipStream_t stream) {
  hipError_t e = launch_doc_stats(a, stream);
  if (e != hipSuccess) return e;
  return launch_final(a, stream);
}

}  // namespace br
