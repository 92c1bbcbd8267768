// Split-key merge of the final-query rows, as a per-workgroup body: the attention path launches
// it as attn_merge_kernel, the ranking path alongside the readout's partial kernel (the two are
// independent, so one launch serves both).
#pragma once

#include "device_common.h"
#include "plan.h"

namespace br {

// Workgroups one (query tile, KV head) pair spreads over (256 threads, one per row and 4 elements).
template <int D>
constexpr int merge_wg_per_tile() { return kRowsPerTile * (D / 4) / 256; }

// Combine split-key partials of one query tile: M = max m_c, L = sum l_c 2^(m_c - M),
// o = sum o_c 2^(m_c - M) / L, accumulated in one pass with a running maximum.  One thread
// per (row, 4 head-dim elements); a workgroup covers 256 such units, so one (query tile, KV
// head) spreads over 128 * D / 4 / 256 workgroups.  Chunks are visited U at a time so their
// loads are in flight together (U is chosen per kernel by its register budget); the sums are
// added in chunk order whatever U is, so the result is deterministic and the same in both
// kernels.
template <int D, int U = 8>
__device__ __forceinline__ void attn_merge_block(int block, uint16_t* __restrict__ O, float* __restrict__ lse,
                                                 const MergeItem* __restrict__ merges, const float* __restrict__ part_o,
                                                 const float* __restrict__ part_ml, int Hq, int Hkv, int G,
                                                 int q_row_base, float sink_log2) {
  constexpr int CH = D / 4;                          // 4-element units per row
  constexpr int WG_PER_TILE = kRowsPerTile * CH / 256;
  const int tile = block / WG_PER_TILE, part = block % WG_PER_TILE;
  const int g = tile % Hkv;
  const MergeItem mi = merges[tile / Hkv];
  const int unit = part * 256 + threadIdx.x;
  const int rho = unit / CH, ch = unit % CH;
  const int tok = mi.row0 + rho / G, h = g * G + rho % G;  // token-major rows
  if (tok >= mi.row_limit) return;
  const int64_t stride = int64_t(Hkv) * kRowsPerTile;  // rows between consecutive slots
  const int64_t row = (int64_t(mi.slot0) * Hkv + g) * kRowsPerTile + rho;
  const float2* ml = reinterpret_cast<const float2*>(part_ml);
  const int n = mi.nslots;
  // One pass with a running maximum: chunk c scales the state by 2^(M - M') and adds its own
  // partials with weight 2^(m_c - M').  Eight chunks' loads are issued together per round.
  float M = -INFINITY, L = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  // Explicit fused multiply-adds: the body is inlined into two kernels (the attention path's
  // merge and the ranking step's merge with the readout), and must round the same in both.
  auto add = [&](float2 v, f32x4_t o) {
    const float Mn = fmaxf(M, v.x);
    if (Mn == -INFINITY) return;  // nothing seen yet
    const float a = fast_exp2(M - Mn), wgt = fast_exp2(v.x - Mn);
    L = fmaf(v.y, wgt, L * a);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, o[e], acc[e] * a);
    M = Mn;
  };
  for (int c = 0; c < n; c += U) {
    float2 v[U];
    f32x4_t o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u < n) {
        v[u] = ml[row + (c + u) * stride];
        o[u] = *reinterpret_cast<const f32x4_t*>(part_o + (row + (c + u) * stride) * D + ch * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c + u < n) add(v[u], o[u]);
  }
  const float inv = 1.f / (L + fast_exp2(sink_log2 - M));  // the sink slot adds exp(b) / 2^M; 0 when b = -inf
  const u32x2_t v = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2_t*>(O + (int64_t(tok - q_row_base) * Hq + h) * D + ch * 4) = v;
  if (lse && ch == 0) lse[int64_t(tok - q_row_base) * Hq + h] = (M + __log2f(L)) * kLn2;
}

}  // namespace br
