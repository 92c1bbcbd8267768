// Block-sparse prefill attention for BlockRank prompts on gfx950 (MI355X).
//
// Computes softmax(Q K^T * scale + M) V where M allows: instruction rows -> instruction keys
// causally; document rows -> the whole instruction plus their own document causally; final
// query rows -> everything before the query plus the query causally (BlockRank summary,
// section 3.4 "Blockwise Structured Attention"; blog, block mask with causal diagonal blocks C;
// BlockSearch section 3.2 for the causal reading of the diagonal blocks).  The host plan lists
// only allowed (row tile, key range) pairs; this kernel never visits a forbidden block.
//
// Row token indices address Q, O and lse relative to q_row_base (0 for whole prompts; the corpus
// length when only query rows over a cached corpus are computed).
//
// Work item = 128 (token, head) rows: TM = 128 / G consecutive tokens of the G query heads
// that share one KV head (grouped-query packing), so each K/V tile staged in LDS serves G
// heads.  Wave w owns 32 rows.  Per 64-key tile:
//   S^T = K Q^T   with v_mfma_f32_32x32x16_bf16 (keys on M, query rows on N), so every lane
//                 holds one query row and 32 of the tile's keys: row max/sum need only one
//                 cross-half exchange (v_permlane32_swap);
//   online softmax in fp32 (log2 domain, exp2), lazy rescaling of the accumulator;
//   O^T += V^T P^T with P rounded to bf16; V is staged row-major and its transposed MFMA
//                 fragments come from transposing LDS reads (ds_read_b64_tr_b16).
//
// The kernel is persistent: each workgroup serves one KV head and runs its share of the item
// list (a host-side list schedule).  Tiles stream through one software pipeline across item
// boundaries: while a tile is computed, the next tile's K/V (on an item's last tile, the next
// item's first tile) is loaded into registers, one load per two S^T MFMAs, then written to the
// other LDS buffer.  Loads and stores go through buffer resources sized to the valid rows, so
// rows past a range end read as zero and writes past a tile's last token are dropped by the
// hardware.
//
// Q and O move as whole rows (1 KB per wave instruction over 8 full cache lines, instead of
// 32 B from each of 32 rows) and are redistributed through LDS: the tile buffer the item's
// last tile used is free until the next item's second tile.  Each wave passes the next item's
// Q rows (loaded once the last tile's S^T is formed) into MFMA fragments through its own 32
// rows of that buffer, then this item's normalised output rows the other way.  Query rows of long prompts are split over key
// chunks; their fp32 partials (m, l, o) are combined by attn_merge_kernel.
#include "attn_merge.h"
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
                                                       const int32_t* __restrict__ ranges, float* __restrict__ part_o,
                                                       float* __restrict__ part_ml, int Hq, int Hkv, float scale_log2,
                                                       int q_row_base) {
  constexpr int TM = kRowsPerTile / G;  // tokens per tile
  constexpr int BN = kKeyTile;          // keys per LDS tile
  constexpr int NKB = BN / 32;          // 32-key MFMA blocks per tile
  constexpr int KROW = D + 8;           // K row stride in LDS (elements): +16 B breaks bank aliasing
  // V row stride in LDS (elements): 4 or 12 (mod 16) 16-byte units, so the 4 rows x 4 units that
  // one half-wave of a transposing read touches fall in 16 different bank groups.
  constexpr int VROW = D == 128 ? 160 : 96;
  static_assert(VROW >= D && ((VROW / 8) % 16 == 4 || (VROW / 8) % 16 == 12), "V row stride");
  constexpr int DSTEPS = D / 16;        // MFMA k-steps over the head dimension
  constexpr int DBLK = D / 32;          // 32-wide output blocks over the head dimension
  constexpr int KCH = D / 8;            // 16-byte chunks per K/V row
  constexpr int KROWS_PER_PASS = 256 / KCH;
  constexpr int KPASS = BN / KROWS_PER_PASS;

  // LDS buffer b holds K tile b (BN x KROW) followed by V tile b (BN x VROW), both row-major.
  // Between an item's last tile and the next item's second tile, the buffer the last tile used
  // is free and redistributes Q and O rows ([row][D + 8], 32 rows per wave).
  constexpr int KBUF = BN * KROW;
  constexpr int TILE = KBUF + BN * VROW;
  __shared__ __align__(16) uint16_t skv[2][TILE];

  const int g = blockIdx.x % Hkv;
  const int wg = blockIdx.x / Hkv;
  const int it_begin = ranges[wg], it_end = ranges[wg + 1];
  if (it_begin >= it_end) return;  // uniform per workgroup

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, n = lane & 31, half = lane >> 5;
  const int rho = w * 32 + n;  // this lane's row within the tile
  const int hh = rho / TM, tt = rho % TM;
  const int h = g * G + hh;
  const int q_stride = Hq * D, kv_stride = Hkv * D;  // elements between consecutive tokens

  // Per-lane byte offsets inside a row block (Q, O) or a key tile (K, V).
  const uint32_t q_off = uint32_t((tt * q_stride + hh * D + 8 * half) * 2);
  const int kcc = tid % KCH, kr0 = tid / KCH;  // K and V: 16-byte chunk and first row of this thread
  const uint32_t k_off = uint32_t((kr0 * kv_stride + 8 * kcc) * 2);
  // P.V A-operand reads (transposing, see lds_read_tr16): in each 16-lane group (s = lane % 16,
  // head-dim half dh = (lane / 16) % 2, key half `half`) lane s points at key 4 half + s / 4 and
  // head-dim element 16 dh + 4 (s % 4) of a block; blocks differ by compile-time offsets.
  const int vs = lane & 15, vdh = (lane >> 4) & 1;
  const int v_lane = KBUF + (4 * half + (vs >> 2)) * VROW + 16 * vdh + 4 * (vs & 3);

  // Q fragments: B operand of S^T = K Q^T (row n, head-dim elements 16 s + 8 half .. +8).
  // Resource over a tile's valid rows of a [T, Hq, D] tensor, based at its first row and head.
  auto row_rsrc = [&](const uint16_t* base, const AttnItem& it) {
    const int rows = min(TM, it.row_limit - it.row0);
    return make_rsrc(base + (int64_t(it.row0 - q_row_base) * Hq + g * G) * D, rows * q_stride * 2);
  };
  u32x4_t qf[DSTEPS];
  auto load_q = [&](const AttnItem& it, u32x4_t* dst) {
    const rsrc_t r = row_rsrc(Q, it);
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) dst[s] = buf_load16(r, q_off + 32 * s);
  };
  // The same rows loaded coalesced: instruction s of wave w reads QRI whole rows (1 KB, 8 full
  // cache lines) instead of 32 B from each of 32 rows; the fragments are then redistributed
  // through LDS ([row][QROW]).  Lane l takes chunk l % KCH of row 32 w + QRI s + l / KCH.
  constexpr int QROW = D + 8;        // staged Q row stride (elements): same bank pattern as K
  constexpr int QRI = 512 / D;       // rows per coalesced instruction
  static_assert(kRowsPerTile * QROW <= TILE && QRI * DSTEPS == kRowsPerWave, "Q staging fits a tile buffer");
  auto load_q_rows = [&](const AttnItem& it, bool valid) {
    const rsrc_t r = valid ? row_rsrc(Q, it) : make_rsrc(Q, 0);  // zero bytes: reads nothing
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) {
      const int rr = 32 * w + QRI * s + lane / KCH;
      qf[s] = buf_load16(r, uint32_t(((rr % TM) * q_stride + (rr / TM) * D + 8 * (lane % KCH)) * 2));
    }
  };
  auto stage_q_rows = [&](uint16_t* st) {
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s)
      *reinterpret_cast<u32x4_t*>(&st[(32 * w + QRI * s + lane / KCH) * QROW + 8 * (lane % KCH)]) = qf[s];
  };
  auto read_q_frags = [&](const uint16_t* st) {
#pragma unroll
    for (int s = 0; s < DSTEPS; ++s) qf[s] = load16(&st[rho * QROW + 16 * s + 8 * half]);
  };

  // ---- global -> registers -> LDS staging of one K/V tile ----
  // KCH adjacent threads load one key row of K and of V (coalesced 256-byte reads) and write it
  // to the same row of the LDS tiles.
  u32x4_t kreg[KPASS], vreg[KPASS];
  // The next tile's loads are issued one at a time among the current tile's S^T MFMAs: issued
  // together at the top of a tile, the loads of all waves on the CU queue in the texture
  // address unit and each wave's in-order issue stalls behind them.  `next_k`/`next_v` cover
  // the next tile's valid keys (zero bytes when there is none, so the loads read nothing).
  rsrc_t next_k, next_v;
  auto plan_tile = [&](int start, int end) {
    const int keys = min(BN, end - start);
    next_k = make_rsrc(K + int64_t(start) * kv_stride + g * D, keys * kv_stride * 2);
    next_v = make_rsrc(V + int64_t(start) * kv_stride + g * D, keys * kv_stride * 2);
  };
  auto no_tile = [&]() {
    next_k = make_rsrc(K, 0);
    next_v = make_rsrc(V, 0);
  };
  constexpr int LOAD_STEPS = 2 * KPASS;
  auto load_step = [&](int j) {
    const int p = j >> 1;
    const uint32_t off = k_off + p * KROWS_PER_PASS * kv_stride * 2;
    if (j & 1)
      vreg[p] = buf_load16(next_v, off);
    else
      kreg[p] = buf_load16(next_k, off);
  };
  auto load_tile = [&](int start, int end) {
    plan_tile(start, end);
#pragma unroll
    for (int j = 0; j < LOAD_STEPS; ++j) load_step(j);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < KPASS; ++p) {
      const int row = kr0 + p * KROWS_PER_PASS;
      *reinterpret_cast<u32x4_t*>(&skv[buf][row * KROW + 8 * kcc]) = kreg[p];
      *reinterpret_cast<u32x4_t*>(&skv[buf][KBUF + row * VROW + 8 * kcc]) = vreg[p];
    }
  };

  // Key tile i of an item: the unmasked range's tiles come first, then the causal range's.
  auto n_unmasked = [](const AttnItem& it) { return it.a_end > it.a_start ? (it.a_end - it.a_start + BN - 1) / BN : 0; };
  auto n_tiles = [&](const AttnItem& it) {
    return n_unmasked(it) + (it.b_end > it.b_start ? (it.b_end - it.b_start + BN - 1) / BN : 0);
  };
  auto tile_start = [&](const AttnItem& it, int nA, int i) { return i < nA ? it.a_start + i * BN : it.b_start + (i - nA) * BN; };
  auto tile_end = [&](const AttnItem& it, int nA, int i) { return i < nA ? it.a_end : it.b_end; };

  f32x16_t o[DBLK];
  float m_run, l_run;

  // One tile: S^T, mask, online softmax, O^T += V^T P^T.  `row_tok` is this lane's token.
  // `after_s` runs once the S^T MFMAs have consumed the Q fragments (on an item's last tile it
  // loads the next item's Q rows into them).
  auto compute = [&](int buf, int start, int end, bool causal, int row0, int row_tok, bool first, auto&& after_s) {
    f32x16_t s[NKB];
    static_assert(NKB * DSTEPS == 2 * LOAD_STEPS, "one next-tile load per two S^T MFMAs");
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16_t{};
      const uint16_t* kp = &skv[buf][(kb * 32 + n) * KROW + 8 * half];
#pragma unroll
      for (int st = 0; st < DSTEPS; ++st) {
        s[kb] = mfma32(load16(kp + 16 * st), qf[st], s[kb]);
        if (st & 1) load_step((kb * DSTEPS + st) >> 1);
      }
    }
    // Instruction order for the scheduler: (2 LDS reads, 2 MFMAs, 1 global load) repeated.
#pragma unroll
    for (int j = 0; j < LOAD_STEPS; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    after_s();
    // Mask only tiles that cross the range end or the causal diagonal of some row.  Register r of
    // block kb holds key start + 32 kb + 8 (r / 4) + 4 half + r % 4.
    if ((start + BN > end) || (causal && start + BN - 1 > row0)) {
      const int lim = (causal ? min(end, row_tok + 1) : end) - start - 4 * half;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = (kb * 32 + 8 * (r >> 2) + (r & 3)) < lim ? s[kb][r] : -INFINITY;
    }
    float mt = s[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = max_halves(mt) * scale_log2;
    if (first) {
      m_run = mt;  // the accumulator is still zero: nothing to rescale
    } else {
      const bool need = mt > m_run + kRescaleSlack;
      if (__any(need)) {
        const float m_new = need ? mt : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DBLK; ++b) o[b] *= alpha;
      }
    }
    const float mu = m_run == -INFINITY ? 0.f : m_run;
    uint32_t pk[NKB][8];
    float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // four partial row sums shorten the add chain
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[kb][r], scale_log2, -mu));
        const float p1 = fast_exp2(fmaf(s[kb][r + 1], scale_log2, -mu));
        pk[kb][r >> 1] = pack_bf16x2(p0, p1);
        lsum[(r >> 1) & 3] += p0 + p1;
      }
    l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    // O^T += V^T P^T, 16 keys per MFMA.  Lane half h of P holds keys 16 m + 4 h + 0..3 and
    // 16 m + 8 + 4 h + 0..3 of block kb (the S^T accumulator order); the two transposing reads
    // give the V^T fragment the same key order.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const u32x4_t pv = {pk[kb][4 * m], pk[kb][4 * m + 1], pk[kb][4 * m + 2], pk[kb][4 * m + 3]};
        const uint16_t* vp = &skv[buf][v_lane + (32 * kb + 16 * m) * VROW];
#pragma unroll
        for (int b = 0; b < DBLK; ++b) {
          const u32x2_t lo = lds_read_tr16(vp + 32 * b), hi = lds_read_tr16(vp + 8 * VROW + 32 * b);
          o[b] = mfma32(u32x4_t{lo[0], lo[1], hi[0], hi[1]}, pv, o[b]);
        }
      }
  };

  // Pipeline prologue: the first item's Q and first tile.
  AttnItem cur = items[it_begin];
  load_q(cur, qf);
  {
    const int nA = n_unmasked(cur);
    load_tile(tile_start(cur, nA, 0), tile_end(cur, nA, 0));
  }
  store_tile(0);
  __syncthreads();
  int buf = 0;

  for (int it = it_begin; it < it_end; ++it) {
    const bool more = it + 1 < it_end;
    const AttnItem nxt = items[more ? it + 1 : it];
    const int nA = n_unmasked(cur), nt = n_tiles(cur);
    const int row_tok = cur.row0 + tt;
#pragma unroll
    for (int b = 0; b < DBLK; ++b) o[b] = f32x16_t{};
    m_run = -INFINITY;
    l_run = 0.f;

    // Every tile prefetches the next one: the item's next tile, or on the last tile the next
    // item's first tile.  The last tile is written out separately: it also loads the next item's
    // Q rows, so that the compiler sees those loads on that path only.
    for (int i = 0; i + 1 < nt; ++i) {
      plan_tile(tile_start(cur, nA, i + 1), tile_end(cur, nA, i + 1));
      compute(buf, tile_start(cur, nA, i), tile_end(cur, nA, i), i >= nA, cur.row0, row_tok, i == 0, [] {});
      store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    if (more) {
      const int nA_next = n_unmasked(nxt);
      plan_tile(tile_start(nxt, nA_next, 0), tile_end(nxt, nA_next, 0));
    } else {
      no_tile();
    }
    compute(buf, tile_start(cur, nA, nt - 1), tile_end(cur, nA, nt - 1), nt - 1 >= nA, cur.row0, row_tok, nt == 1,
            [&] { load_q_rows(nxt, more); });
    if (more) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    // The buffer the last tile used is free until the next item's second tile.  Each wave uses
    // its own 32 rows of it ([row][QROW]) to redistribute the next item's Q rows and then this
    // item's outputs; a wave's LDS operations complete in order, so only the barrier at the end
    // of the epilogue is needed.  (Done after the last item too, on zero rows, so that every
    // path reaches the next tile with the fragments read from LDS and the compiler adds no
    // memory-counter waits there.)
    uint16_t* const xbuf = skv[buf ^ 1];
    stage_q_rows(xbuf);
    read_q_frags(xbuf);

    // Epilogue: normalise and store this item's rows (or its split-key partials).
    const float l_tot = l_run + other_half(l_run);
    if (cur.slot < 0) {
      const float inv = 1.f / l_tot;
      const rsrc_t ro = row_rsrc(O, cur);  // rows past the tile's last token are dropped
#pragma unroll
      for (int b = 0; b < DBLK; ++b)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          // Lane half 0 holds head-dim elements 8j..8j+3 and half 1 holds 8j+4..8j+7 of each
          // 8-element group j; swapping one group pair across halves gives every lane 8
          // contiguous outputs: half 0 stages group 2t, half 1 stages group 2t+1.
          const int j0 = 2 * t, j1 = 2 * t + 1;
          const uint32_t a0 = pack_bf16x2(o[b][4 * j0] * inv, o[b][4 * j0 + 1] * inv);
          const uint32_t a1 = pack_bf16x2(o[b][4 * j0 + 2] * inv, o[b][4 * j0 + 3] * inv);
          const uint32_t b0 = pack_bf16x2(o[b][4 * j1] * inv, o[b][4 * j1 + 1] * inv);
          const uint32_t b1 = pack_bf16x2(o[b][4 * j1 + 2] * inv, o[b][4 * j1 + 3] * inv);
          const uint32_t x0 = half ? a0 : b0, x1 = half ? a1 : b1;
          const auto r0 = __builtin_amdgcn_permlane32_swap(x0, x0, false, false);
          const auto r1 = __builtin_amdgcn_permlane32_swap(x1, x1, false, false);
          const u32x4_t v = half ? u32x4_t{r0[0], r1[0], b0, b1} : u32x4_t{a0, a1, r0[1], r1[1]};
          *reinterpret_cast<u32x4_t*>(&xbuf[rho * QROW + 32 * b + 16 * t + 8 * half]) = v;
        }
      if (lse && half == 0 && row_tok < cur.row_limit)
        lse[int64_t(row_tok - q_row_base) * Hq + h] = (m_run + __log2f(l_tot)) * kLn2;
      // Whole-row stores of this wave's rows: instruction s writes QRI rows (1 KB, 8 full
      // cache lines), lane l chunk l % KCH of row 32 w + QRI s + l / KCH.
#pragma unroll
      for (int s2 = 0; s2 < DSTEPS; ++s2) {
        const int rr = 32 * w + QRI * s2 + lane / KCH;
        buf_store16(load16(&xbuf[rr * QROW + 8 * (lane % KCH)]), ro,
                    uint32_t(((rr % TM) * q_stride + (rr / TM) * D + 8 * (lane % KCH)) * 2));
      }
    } else {
      const int64_t sl = int64_t(cur.slot) * Hkv + g;
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
    __syncthreads();  // the freed buffer takes the tile after the next item's first
    if (more) cur = nxt;
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(uint16_t* __restrict__ O, float* __restrict__ lse,
                                                         const MergeItem* __restrict__ merges,
                                                         const float* __restrict__ part_o,
                                                         const float* __restrict__ part_ml, int Hq, int Hkv, int G,
                                                         int q_row_base) {
  attn_merge_block<D>(blockIdx.x, O, lse, merges, part_o, part_ml, Hq, Hkv, G, q_row_base);
}

template <int D, int G>
static hipError_t launch_attn_t(const AttnLaunch& a, hipStream_t stream) {
  if (a.n_items > 0) {
    const dim3 grid(unsigned(a.wg_per_head * a.num_kv_heads));
    if (a.ev_start) {
      hipError_t e = hipEventRecord(a.ev_start, stream);
      if (e != hipSuccess) return e;
    }
    attn_fwd_kernel<D, G><<<grid, 256, 0, stream>>>(a.Q, a.K, a.V, a.O, a.lse, a.items, a.ranges, a.part_o, a.part_ml,
                                                    a.num_q_heads, a.num_kv_heads, a.scale_log2, a.q_row_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev_stop) {
      e = hipEventRecord(a.ev_stop, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (a.n_merges > 0 && !a.defer_merge) {
    const dim3 grid(unsigned(a.n_merges * a.num_kv_heads * merge_wg_per_tile<D>()));
    attn_merge_kernel<D><<<grid, 256, 0, stream>>>(a.O, a.lse, a.merges, a.part_o, a.part_ml, a.num_q_heads,
                                                   a.num_kv_heads, G, a.q_row_base);
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
