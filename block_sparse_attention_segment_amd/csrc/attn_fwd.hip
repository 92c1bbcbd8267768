// Block-sparse prefill attention for BlockRank prompts on gfx950 (MI355X).
//
// Computes softmax(Q K^T * scale + M) V where M allows: instruction rows -> instruction keys
// causally; document rows -> the whole instruction plus their own document causally; final
// query rows -> everything before the query plus the query causally (BlockRank summary,
// section 3.4 "Blockwise Structured Attention"; blog, block mask with causal diagonal blocks C;
// BlockSearch section 3.2 for the causal reading of the diagonal blocks).  The host plan lists
// only allowed (row tile, key range) pairs; this kernel never visits a forbidden block.
//
// Work item = 128 (token, head) rows: TM = 128 / G consecutive tokens of the G query heads
// that share one KV head (grouped-query packing), so each K/V tile staged in LDS serves G
// heads.  Wave w owns 32 rows.  Per 64-key tile:
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16 (keys on M, query rows on N), so every lane
//                 holds one query row and 32 of the tile's keys: row max/sum need only one
//                 cross-half exchange (v_permlane32_swap);
//   online softmax in fp32 (log2 domain, exp2), lazy rescaling of the accumulator;
//   O^T += V^T P^T with P rounded to bf16, V staged transposed in LDS.
// K/V tiles are double-buffered in LDS with the next tile prefetched into registers.
// Query rows of long prompts are split over key chunks; their fp32 partials (m, l, o) are
// combined by attn_merge_kernel with the usual log-sum-exp algebra.
#include "device_common.h"
#include "launch.h"
#include "plan.h"

namespace br {

// Accumulator rescaling is skipped until the running maximum grows by more than this many
// log2 units, so probabilities stay <= 2^8 before normalisation (exact in fp32 and bf16 range).
constexpr float kRescaleSlack = 8.0f;

template <int D, int G>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                                                       float* __restrict__ lse, const AttnItem* __restrict__ items,
                                                       float* __restrict__ part_o, float* __restrict__ part_ml, int Hq,
                                                       int Hkv, float scale_log2) {
  constexpr int TM = kRowsPerTile / G;  // tokens per tile
  constexpr int BN = kKeyTile;          // keys per LDS tile
  constexpr int KROW = D + 8;           // K row stride in LDS (elements): +16 B breaks bank aliasing
  constexpr int VROW = BN + 8;          // transposed-V row stride in LDS (elements)
  constexpr int DSTEPS = D / 16;        // MFMA k-steps over the head dimension
  constexpr int DBLK = D / 32;          // 32-wide output blocks over the head dimension
  constexpr int KCH = D / 8;            // 16-byte chunks per K/V row
  constexpr int KROWS_PER_PASS = 256 / KCH;
  constexpr int KPASS = BN / KROWS_PER_PASS;
  constexpr int VGROUPS = BN / 4;       // groups of 4 keys in a V tile

  __shared__ __align__(16) uint16_t sk[2][BN * KROW];
  __shared__ __align__(16) uint16_t sv[2][D * VROW];

  const int g = blockIdx.x % Hkv;
  const AttnItem* itp = items + blockIdx.x / Hkv;
  const int row0 = itp->row0, row_limit = itp->row_limit, a_start = itp->a_start, a_end = itp->a_end;
  const int b_start = itp->b_start, b_end = itp->b_end, slot = itp->slot;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, half = lane >> 5;
  const int rho = w * 32 + n;  // this lane's row within the tile
  const int hh = rho / TM, tt = rho % TM;
  const int h = g * G + hh;
  const int row_tok = row0 + tt;
  const bool row_ok = row_tok < row_limit;
  const int64_t q_stride = int64_t(Hq) * D, kv_stride = int64_t(Hkv) * D;

  // Q fragments: B operand of S^T = K Q^T (row n, head-dim elements 16 s + 8 half .. +8).
  u32x4_t qf[DSTEPS];
  {
    const uint16_t* qp = Q + int64_t(row_tok) * q_stride + int64_t(h) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) qf[s] = row_ok ? load16(qp + 16 * s) : u32x4_t{0, 0, 0, 0};
  }

  const int nA = a_end > a_start ? (a_end - a_start + BN - 1) / BN : 0;
  const int nB = b_end > b_start ? (b_end - b_start + BN - 1) / BN : 0;
  const int nt = nA + nB;

  // ---- global -> registers -> LDS staging of one K/V tile ----
  const int kcc = tid % KCH, kr0 = tid / KCH;  // K: 16-byte chunk and first row of this thread
  const int vdc = tid % KCH, vkg = tid / KCH;  // V: 8-element head-dim chunk and 4-key group
  u32x4_t kreg[KPASS], vreg[4];
  auto load_tile = [&](int start, int end) {
    const uint16_t* kb = K + int64_t(g) * D + 8 * kcc;
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int j = start + kr0 + p * KROWS_PER_PASS;
      kreg[p] = j < end ? load16(kb + int64_t(j) * kv_stride) : u32x4_t{0, 0, 0, 0};
    }
    if (vkg < VGROUPS) {
      const uint16_t* vb = V + int64_t(g) * D + 8 * vdc;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = start + 4 * vkg + c;
        vreg[c] = j < end ? load16(vb + int64_t(j) * kv_stride) : u32x4_t{0, 0, 0, 0};
      }
    }
  };
  // V is stored transposed (row = head-dim element, column = key).  Within each 16-key group
  // the keys are stored in the order 0-3, 8-11, 4-7, 12-15, which makes the 8 keys one lane
  // feeds to a P.V MFMA contiguous; 16-byte column chunks are XOR-swizzled by (d / 16) % 8.
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p)
      *reinterpret_cast<u32x4_t*>(&sk[buf][(kr0 + p * KROWS_PER_PASS) * KROW + 8 * kcc]) = kreg[p];
    if (vkg < VGROUPS) {
      const int pos = 16 * (vkg >> 2) + 8 * (vkg & 1) + 4 * ((vkg >> 1) & 1);
      const int chunk = pos >> 3, sub = pos & 7;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w0 = vreg[0][u], w1 = vreg[1][u], w2 = vreg[2][u], w3 = vreg[3][u];
        const u32x2_t even = {(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16)};
        const u32x2_t odd = {(w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        const int d0 = 8 * vdc + 2 * u, d1 = d0 + 1;
        *reinterpret_cast<u32x2_t*>(&sv[buf][d0 * VROW + 8 * (chunk ^ ((d0 >> 4) & 7)) + sub]) = even;
        *reinterpret_cast<u32x2_t*>(&sv[buf][d1 * VROW + 8 * (chunk ^ ((d1 >> 4) & 7)) + sub]) = odd;
      }
    }
  };
  // Key tile i: the unmasked range's tiles come first, then the causal range's.
  auto tile_start = [&](int i) { return i < nA ? a_start + i * BN : b_start + (i - nA) * BN; };
  auto tile_end = [&](int i) { return i < nA ? a_end : b_end; };

  f32x16_t o[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b) o[b] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](int buf, int start, int end, bool causal) {
    // S^T for keys start .. start+63 (two 32-key blocks) against this wave's 32 rows.
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16_t{};
      const uint16_t* kp = &sk[buf][(kb * 32 + n) * KROW + 8 * half];
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) s[kb] = mfma32(load16(kp + 16 * st), qf[st], s[kb]);
    }
    // Mask only tiles that cross the range end or the causal diagonal of some row.
    const bool need_mask = (start + BN > end) || (causal && start + BN - 1 > row0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = start + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool ok = j < end && (!causal || j <= row_tok);
          s[kb][r] = ok ? s[kb][r] : -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = max_halves(mt) * scale_log2;
    const bool need = mt > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < DBLK; ++b) o[b] *= alpha;
    }
    const float mu = m_run == -INFINITY ? 0.f : m_run;
    uint32_t pk[2][8];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[kb][r], scale_log2, -mu));
        const float p1 = fast_exp2(fmaf(s[kb][r + 1], scale_log2, -mu));
        lsum += p0 + p1;
        pk[kb][r >> 1] = pack_bf16x2(p0, p1);
      }
    l_run += lsum;
    // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x4_t pv = {pk[kb][4 * m], pk[kb][4 * m + 1], pk[kb][4 * m + 2], pk[kb][4 * m + 3]};
        const int cpos = 2 * (2 * kb + m) + half;
#pragma unroll
        for (int b = 0; b < DBLK; ++b) {
          const int d = 32 * b + n;
          const u32x4_t vf = load16(&sv[buf][d * VROW + 8 * (cpos ^ ((d >> 4) & 7))]);
          o[b] = mfma32(vf, pv, o[b]);
        }
      }
  };

  load_tile(tile_start(0), tile_end(0));
  store_tile(0);
  __syncthreads();
  for (int i = 0; i < nt; ++i) {
    const bool has_next = i + 1 < nt;
    if (has_next) load_tile(tile_start(i + 1), tile_end(i + 1));
    compute(i & 1, tile_start(i), tile_end(i), i >= nA);
    if (has_next) store_tile((i + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + other_half(l_run);
  if (slot < 0) {
    if (row_ok) {
      const float inv = 1.f / l_tot;
      uint16_t* op = O + int64_t(row_tok) * q_stride + int64_t(h) * D + 4 * half;
#pragma unroll
      for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x2_t v = {pack_bf16x2(o[b][4 * j] * inv, o[b][4 * j + 1] * inv),
                             pack_bf16x2(o[b][4 * j + 2] * inv, o[b][4 * j + 3] * inv)};
          *reinterpret_cast<u32x2_t*>(op + 32 * b + 8 * j) = v;
        }
      if (lse && half == 0) lse[int64_t(row_tok) * Hq + h] = (m_run + __log2f(l_tot)) * kLn2;
    }
  } else {
    const int64_t sl = int64_t(slot) * Hkv + g;
    float* po = part_o + (sl * kRowsPerTile + rho) * D + 4 * half;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4_t*>(po + 32 * b + 8 * j) =
            f32x4_t{o[b][4 * j], o[b][4 * j + 1], o[b][4 * j + 2], o[b][4 * j + 3]};
    if (half == 0) {
      part_ml[(sl * kRowsPerTile + rho) * 2] = m_run;
      part_ml[(sl * kRowsPerTile + rho) * 2 + 1] = l_tot;
    }
  }
}

// Combine split-key partials of one query tile: M = max m_c, L = sum l_c 2^(m_c - M),
// o = sum o_c 2^(m_c - M) / L.  One thread per (row, 8 head-dim elements); a workgroup covers
// 256 such units, so one (query tile, KV head) spreads over 128 * D / 8 / 256 workgroups.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(uint16_t* __restrict__ O, float* __restrict__ lse,
                                                         const MergeItem* __restrict__ merges,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int Hq, int Hkv, int G) {
  constexpr int CH = D / 8;                          // 8-element chunks per row
  constexpr int WG_PER_TILE = kRowsPerTile * CH / 256;
  const int tile = blockIdx.x / WG_PER_TILE, part = blockIdx.x % WG_PER_TILE;
  const int g = tile % Hkv;
  const MergeItem mi = merges[tile / Hkv];
  const int unit = part * 256 + threadIdx.x;
  const int rho = unit / CH, ch = unit % CH;
  const int TM = kRowsPerTile / G;
  const int tok = mi.row0 + rho % TM, h = g * G + rho / TM;
  if (tok >= mi.row_limit) return;
  const int64_t stride = int64_t(Hkv) * kRowsPerTile;  // rows between consecutive slots
  const int64_t row = (int64_t(mi.slot0) * Hkv + g) * kRowsPerTile + rho;
  float M = -INFINITY;
  for (int c = 0; c < mi.nslots; ++c) M = fmaxf(M, part_ml[(row + c * stride) * 2]);
  float L = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < mi.nslots; ++c) {
    const int64_t r = row + c * stride;
    const float wgt = fast_exp2(part_ml[r * 2] - M);
    L += part_ml[r * 2 + 1] * wgt;
    const f32x4_t* po = reinterpret_cast<const f32x4_t*>(part_o + r * D + ch * 8);
    const f32x4_t v0 = po[0], v1 = po[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += wgt * v0[e];
      acc[4 + e] += wgt * v1[e];
    }
  }
  const float inv = 1.f / L;
  const u32x4_t v = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  *reinterpret_cast<u32x4_t*>(O + (int64_t(tok) * Hq + h) * D + ch * 8) = v;
  if (lse && ch == 0) lse[int64_t(tok) * Hq + h] = (M + __log2f(L)) * kLn2;
}

template <int D, int G>
static hipError_t launch_attn_t(const AttnLaunch& a, hipStream_t stream) {
  if (a.n_items > 0) {
    const dim3 grid(unsigned(a.n_items * a.num_kv_heads));
    if (a.ev_start) {
      hipError_t e = hipEventRecord(a.ev_start, stream);
      if (e != hipSuccess) return e;
    }
    attn_fwd_kernel<D, G><<<grid, 256, 0, stream>>>(a.Q, a.K, a.V, a.O, a.lse, a.items, a.part_o, a.part_ml,
                                                    a.num_q_heads, a.num_kv_heads, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev_stop) {
      e = hipEventRecord(a.ev_stop, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (a.n_merges > 0) {
    const dim3 grid(unsigned(a.n_merges * a.num_kv_heads * (kRowsPerTile * (D / 8) / 256)));
    attn_merge_kernel<D><<<grid, 256, 0, stream>>>(a.O, a.lse, a.merges, a.part_o, a.part_ml, a.num_q_heads,
                                                   a.num_kv_heads, G);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.num_kv_heads;
  if (a.head_dim == 128) {
    switch (G) {
      case 1: return launch_attn_t<128, 1>(a, stream);
      case 2: return launch_attn_t<128, 2>(a, stream);
      case 4: return launch_attn_t<128, 4>(a, stream);
      case 8: return launch_attn_t<128, 8>(a, stream);
    }
  } else if (a.head_dim == 64) {
    switch (G) {
      case 1: return launch_attn_t<64, 1>(a, stream);
      case 2: return launch_attn_t<64, 2>(a, stream);
      case 4: return launch_attn_t<64, 4>(a, stream);
      case 8: return launch_attn_t<64, 8>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace br
